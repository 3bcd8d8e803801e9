// FP8 (e4m3 x e4m3 -> fp32) GEMMs of the packed QKV projection on the gfx950
// matrix cores: forward x @ W_packed ("96 is enough", "The change": one FP8
// matmul, one launch, one weight read), dX through the cached row-major
// W_packed codes and dW = x^T dQKV (PR #344 page, "Changes": FP8 backward;
// "Where the eight seconds were hiding", "The inventory": the cached
// transposed view serves the backward pass).
//
// All three are C[m][n] = sum_k A[m][k] * B[n][k] with both operands
// K-contiguous in memory, built from v_mfma_scale_f32_32x32x64_f8f6f4 with
// neutral E8M0 scales (a bare loop of it sustains 4.6-4.8 PFLOP/s here,
// against ~3.2-3.9 for the 16x16x128 form).
//
// A block is 8 waves with two roles.  Waves 0-3 (one per SIMD) are the
// matrix waves: 2 x 2 of them (4 x 1 in the fused forward) compute a
// BM x BN tile and never load from global memory.  Waves 4-7 are the copy waves: they fill a ring of three
// LDS stages, K advancing 128 bytes per stage, with direct global-to-LDS
// loads and wait only on their own vector-memory counter.  As that counter
// is per wave, the matrix waves' output stores never hold up the operand
// stream, and the copy waves keep two stages in flight while the matrix
// waves work on the third.  One workgroup barrier per step hands a stage
// over; it carries no memory fence, so no wave waits for stores there.
//
// One load instruction of a copy wave fills 1 KiB = 8 consecutive 128-byte
// LDS rows; lane i lands at physical 16-byte chunk i % 8 of row i / 8 and
// therefore fetches logical chunk (i % 8) ^ (row / 2 % 8): the XOR swizzle
// that spreads the 16 rows of one LDS read phase over all banks.
//
// The MFMA's first operand is fed from B (n rows), its second from A (m
// rows).  The 32x32 result then lands with lane l holding, for each group
// g of four accumulator registers, four consecutive n (8g + 4(l/32) + 0..3)
// of one m (l % 32).  Which k each byte of a lane's 32-byte operand stands
// for does not matter, as both operands use the same assignment.
//
// bf16 outputs (forward, dX, the MLP's) come from persistent kernels, one
// block per CU walking its tiles; a finished 32-row slice of a matrix
// wave's tile is transposed through that wave's own 4 KiB of LDS so that
// every lane stores a 16-byte run of one row.  The forward for head widths
// 64, 96 and 128 also normalises and rotates q and k in that epilogue
// (gemm_qkv_fwd_kernel, below).  dW (K = tokens) reads x8 and g8 as the
// quantiser stores them, token by token, and turns them into MFMA operands
// with transposing LDS reads; it splits K over blocks and writes fp32
// partial sums that a second kernel adds in split order.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace fpr {

typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kBK = 128;  // bytes (= e4m3 elements) of K per step
constexpr int kCopyWaves = 4;
constexpr int kStages = 3;

// Operand formats of the matrix cores' f8f6f4 instructions (the codes of
// their cbsz / blgp fields): OCP E4M3 and OCP E5M2.
constexpr int kFmtE4M3 = 0, kFmtE5M2 = 1;

// A BM x BN tile computed by MW x NW matrix waves (wave w: rows w / NW,
// columns w % NW) and filled by kCopyWaves copy waves; A and B hold codes
// of format FA and FB.
template <int BM, int BN, int MW = 2, int NW = 2, int FA = kFmtE4M3, int FB = kFmtE4M3>
struct TileCfg {
  static constexpr int BM_ = BM, BN_ = BN, FA_ = FA, FB_ = FB;
  static constexpr int MMA = MW * NW, NW_ = NW;
  static constexpr int THREADS = 64 * (MMA + kCopyWaves);
  static constexpr int WM = BM / MW, WN = BN / NW;     // one matrix wave's part
  static constexpr int FM = WM / 32, FN = WN / 32;     // 32x32 fragments per wave
  static constexpr int STAGE_BYTES = (BM + BN) * kBK;  // one K step of A and B rows
  static constexpr int BLOCKS = (BM + BN) / 8;         // 1 KiB DMA blocks per stage
  static constexpr int PER_WAVE = BLOCKS / kCopyWaves;
  static constexpr int A_PER_WAVE = BM / 8 / kCopyWaves;  // a wave's first blocks hold A rows
  static_assert(FM * 32 * MW == BM && FN * 32 * NW == BN, "tile/waves");
  static_assert(BM % 16 == 0, "B rows keep their swizzle key at stage row BM + r");
  static_assert(BLOCKS % kCopyWaves == 0 && (BM / 8) % kCopyWaves == 0, "DMA blocks per wave");
  static_assert(PER_WAVE < 64, "vmcnt range");
};

// Workgroup barrier without a memory fence, after this wave's LDS
// operations are done (the matrix waves' fragment reads, the copy waves'
// tail blanking).  Global stores stay in flight.  The clobber keeps the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Stage rows are 128 bytes, half of the 64 four-byte LDS banks, so rows r
// and r + 1 sit on opposite halves.  A ds_read_b128 phase of 16 lanes reads
// one chunk of 16 consecutive rows; keying the XOR on row / 2 gives those 16
// rows 16 distinct (bank half, chunk) slots, i.e. every bank once.  (Keying
// it on row % 8 repeats each slot for rows r and r + 8: two-way conflicts
// on every fragment read.)
__device__ inline int swz_key(int row) { return (row >> 1) & 7; }
__device__ inline int swz(int row, int chunk) { return row * kBK + ((chunk ^ swz_key(row)) << 4); }

__device__ inline v8i as_v8i(uint4 lo, uint4 hi) {
  v8i r;
  r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
  r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
  return r;
}

// One 32-row MFMA operand for K substep h (64 bytes): lane l takes row
// `row` (= base + l % 32) and the 32 bytes [64h + 32(l/32), +32).
__device__ __forceinline__ v8i lds_frag(const uint8_t* base, int row, int kg, int h) {
  const int c = 4 * h + 2 * kg;
  return as_v8i(*reinterpret_cast<const uint4*>(base + swz(row, c)),
                *reinterpret_cast<const uint4*>(base + swz(row, c + 1)));
}

// ---- token-major operands (dW)
//
// dW = x^T g contracts over tokens, and x8, g8 are stored token by token
// (features contiguous).  The dW stage therefore holds A as 128 token rows
// of 256 feature bytes and B as 128 token rows of 128, and the operands
// reach the MFMA layout through transposing LDS reads: in each 16-lane
// group of ds_read_b64_tr_b8, byte k of lane i comes from byte i % 8 of the
// 8 bytes addressed by lane 2k + i / 8.  Lane r = 2k + e of a group points
// at token t0 + k, features f + 8e, so lane i receives features f + i of
// tokens t0 .. t0 + 7; four such reads give a lane the 32 tokens of its
// K half for one feature row, in the order the other operand uses too.
// Rows are stored in 32-byte segments, segment s of token row t at
// s ^ key(t): the 8 rows one 32-lane read phase touches then fall on 8
// distinct bank octets (A rows span 256 bytes, key t % 8; B rows 128 bytes,
// where rows t and t + 1 already sit on opposite bank halves, key t / 2 % 4).
typedef int v2i_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i_t lds_v2i;

template <int PITCH>
__device__ inline int tok_key(int t) { return PITCH == 256 ? (t & 7) : ((t >> 1) & 3); }
template <int PITCH>
__device__ inline int tok_at(int t, int f) {
  return t * PITCH + (((f >> 5) ^ tok_key<PITCH>(t)) << 5) + (f & 31);
}

// One 32-row operand of K half h: lane l holds feature row f0 + l % 32 and
// the 32 tokens 64h + 32(l / 32) + [0, 32) of the stage.
template <int PITCH>
__device__ __forceinline__ v8i tok_frag(const uint8_t* base, int f0, int lane, int h) {
  const int r = lane & 15;
  const int f = f0 + ((lane >> 4) & 1) * 16 + 8 * (r & 1);
  const int t0 = 64 * h + 32 * (lane >> 5) + (r >> 1);
  v8i out;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const v2i_t x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (lds_v2i*)(base + tok_at<PITCH>(t0 + 8 * q, f)));
    out[2 * q] = x[0];
    out[2 * q + 1] = x[1];
  }
  return out;
}

// The A (rows a0 + l % 32) and B (rows b0 + l % 32) operands of K half h of
// a stage, in either storage.
template <class C, bool TOK>
__device__ __forceinline__ v8i frag_a(const uint8_t* stage, int a0, int lane, int h) {
  if constexpr (TOK) return tok_frag<C::BM_>(stage, a0, lane, h);
  else return lds_frag(stage, a0 + (lane & 31), lane >> 5, h);
}
template <class C, bool TOK>
__device__ __forceinline__ v8i frag_b(const uint8_t* stage, int b0, int lane, int h) {
  if constexpr (TOK) return tok_frag<C::BN_>(stage + C::BM_ * kBK, b0, lane, h);
  else return lds_frag(stage + C::BM_ * kBK, b0 + (lane & 31), lane >> 5, h);
}

// The instruction's first operand is B (format field cbsz), its second A
// (blgp).
template <class C>
__device__ __forceinline__ v16f mfma32(v8i b, v8i a, v16f c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c, C::FB_, C::FA_, 0, 127, 0, 127);
}

// ------------------------------------------------------------ schedule

// The operands and the (tile, K step) pairs a block walks, in order.  Step
// g belongs to the block's tile number ord = g / nk, at K step ks0 + g % nk.
// A split-K block has one tile and a K range.  A persistent block has
// several tiles and all K steps: its group x of P takes the row panels
// m = x, x + P, ... and their tiles in (m, n) order, of which the block
// takes every c-th from the i-th.  With P = 8 and blocks dispatched
// round-robin over the 8 XCDs, group x is one XCD: its blocks work on a
// few row panels at a time that no other XCD touches, so the A rows come
// from memory once and are shared in that XCD's L2.
// An operand is either row-major with leading dimension ld, or blocked
// (blk > 0): blocks of blk rows x 128 bytes of K, as the activation
// quantiser writes them (the tile's rows for that operand divide blk).
// With tok, both operands are token-major instead (dW: K = tokens): the
// row layouts of x8 and g8, blocks of kActRows tokens x kKBlock features,
// lda / ldb = feature blocks per block row.
// Head-aligned column tiles of the forward projection (d > 0; d = 0 means
// tile column c of tile n is packed column 128 n + c).  128-column tile n
// < n_mixed holds the hpt whole Q/K heads n hpt, n hpt + 1, ... (d columns
// each) followed by `fill` columns of V (V columns n fill, ...); later tiles
// hold 128 V columns each, from n_mixed fill on.  The copy waves fetch the
// B rows of each tile in this order, so every matrix wave of a 256 x 128
// tile (64 rows x all 128 columns) sees whole Q/K head rows.
struct ColMap {
  int d, hpt, fill, n_mixed, nqk2, nv;  // head width, heads per tile, V columns
                                        // per mixed tile, mixed tiles, Q|K and V columns
  // packed column of column c (< 128) of tile column n, or -1 (none)
  __host__ __device__ int natural(int n, int c) const {
    if (n < n_mixed) {
      const int hd = hpt * d;
      if (c < hd) {
        const int col = (n * hpt + c / d) * d + c % d;
        return col < nqk2 ? col : -1;
      }
      const int f = n * fill + (c - hd);
      return f < nv ? nqk2 + f : -1;
    }
    const int v = n_mixed * fill + (n - n_mixed) * 128 + c;
    return v < nv ? nqk2 + v : -1;
  }
};

struct Gemm {
  const uint8_t* A;
  int64_t lda;
  const uint8_t* B;
  int64_t ldb;
  int M, N, K, n_tiles;
  int a_blk, b_blk;  // 0: row-major; else block rows
  int tok;
  ColMap cm;         // B row order (forward with the fused norm/RoPE)
};

struct Sched {
  int nk, ks0, steps;
  int single;                 // >= 0: the block's only tile
  int x, P, i, c, n_tiles;    // otherwise: panel group, groups, rank, stride
  __device__ int ord(int g) const { return g / nk; }
  __device__ int tile_of(int o) const {
    if (single >= 0) return single;
    const int k = i + c * o, q = k / n_tiles;
    return (x + P * q) * n_tiles + (k - q * n_tiles);
  }
  __device__ int tile(int g) const { return tile_of(ord(g)); }
  __device__ int ks(int g) const { return ks0 + g - ord(g) * nk; }
};

// ------------------------------------------------------------ copy waves

// Per-lane DMA offsets of one tile: block t of copy wave w covers stage
// rows [8(w + 4t), +8).  Offsets are relative to the tile's first A (resp.
// B) row, with rows past M (resp. N) clamped to the last valid one.
template <class C>
struct CopyState {
  uint32_t off[C::PER_WAVE];
  const uint8_t* Atile;
  const uint8_t* Btile;
  int tile;    // tile the offsets belong to
  int issued;  // steps issued so far
};

// Token-major stage (dW): A block u (< BM / 8) holds token rows 4u .. 4u + 3,
// B block u rows 8u .. 8u + 7; lane j of a block lands at physical 16-byte
// chunk j % (row chunks) of its row and fetches the chunk that tok_at()
// puts there.  Features past the padded width read the last chunk (only
// output rows and columns that are never stored see them).  Offsets are
// from the first token row of the step's 128 within its 256-row block.
template <class C>
__device__ __forceinline__ uint32_t tok_off(int u, int lane, bool is_a, int f0, int fpad) {
  const int pitch = is_a ? C::BM_ : C::BN_, per_row = pitch / 16;
  const int t = u * (1024 / pitch) + lane / per_row, p = lane % per_row;
  const int key = is_a ? tok_key<C::BM_>(t) : tok_key<C::BN_>(t);
  const int f = min(f0 + ((((p >> 1) ^ key)) << 5) + ((p & 1) << 4), fpad - 16);
  return (uint32_t)((((f >> 7) * kActRows + t) << 7) + (f & 127));
}

template <class C>
__device__ __forceinline__ void dma_plan(CopyState<C>& st, const Gemm& gm, int tile, int cw,
                                         int lane) {
  const int m0 = (tile / gm.n_tiles) * C::BM_, n0 = (tile % gm.n_tiles) * C::BN_;
  if (gm.tok) {
#pragma unroll
    for (int t = 0; t < C::PER_WAVE; ++t) {
      const bool is_a = t < C::A_PER_WAVE;
      const int u = cw + kCopyWaves * (is_a ? t : t - C::A_PER_WAVE);
      st.off[t] = is_a ? tok_off<C>(u, lane, true, m0, (int)gm.lda * kBK)
                       : tok_off<C>(u, lane, false, n0, (int)gm.ldb * kBK);
    }
    st.Atile = gm.A;
    st.Btile = gm.B;
    st.tile = tile;
    return;
  }
  const int rl = lane >> 3, p = lane & 7;
  const int64_t ra = gm.a_blk ? kBK : gm.lda, rb = gm.b_blk ? kBK : gm.ldb;
#pragma unroll
  for (int t = 0; t < C::PER_WAVE; ++t) {
    const int row = (cw + kCopyWaves * t) * 8 + rl;
    const uint32_t chunk = (uint32_t)((p ^ swz_key(row)) << 4);
    if (t < C::A_PER_WAVE) {
      st.off[t] = (uint32_t)((min(m0 + row, gm.M - 1) - m0) * ra) + chunk;
    } else if (gm.cm.d) {  // mapped B rows, offsets from B itself (N * ldb < 2^31)
      const int nc = gm.cm.natural(tile % gm.n_tiles, row - C::BM_);
      st.off[t] = (uint32_t)((nc < 0 ? 0 : nc) * rb) + chunk;
    } else {
      st.off[t] = (uint32_t)((min(n0 + row - C::BM_, gm.N - 1) - n0) * rb) + chunk;
    }
  }
  // a blocked operand's tile rows lie inside one block of blk rows (the
  // tile's rows divide blk): block m0 / blk, from its row m0 % blk on
  const int64_t kblocks = (gm.K + kBK - 1) / kBK;
  st.Atile = gm.a_blk ? gm.A + ((int64_t)(m0 / gm.a_blk) * kblocks * gm.a_blk + m0 % gm.a_blk) * kBK
                      : gm.A + (int64_t)m0 * gm.lda;
  st.Btile = gm.cm.d  ? gm.B
             : gm.b_blk ? gm.B + ((int64_t)(n0 / gm.b_blk) * kblocks * gm.b_blk + n0 % gm.b_blk) * kBK
                        : gm.B + (int64_t)n0 * gm.ldb;
  st.tile = tile;
}

// Issue the DMA of the block's next step into its stage.  With KTAIL,
// chunks past K are fetched from inside the row instead and blanked by
// zero_tail() once they have landed.
template <class C, bool KTAIL>
__device__ __forceinline__ void issue_next(CopyState<C>& st, uint8_t* lds, const Gemm& gm,
                                           const Sched& sc, int cw, int lane) {
  const int g = st.issued++;
  const int tile = sc.tile(g);
  if (tile != st.tile) dma_plan<C>(st, gm, tile, cw, lane);
  const int ks = sc.ks(g), k0 = ks * kBK;
  const uint8_t* Ak;
  const uint8_t* Bk;
  if (gm.tok) {  // block row ks / 2, its first or second 128 tokens
    const int64_t half = (int64_t)(ks & 1) * kBK * kBK;
    Ak = st.Atile + (int64_t)(ks >> 1) * gm.lda * kActRows * kBK + half;
    Bk = st.Btile + (int64_t)(ks >> 1) * gm.ldb * kActRows * kBK + half;
  } else {
    Ak = st.Atile + (gm.a_blk ? (int64_t)ks * gm.a_blk * kBK : k0);
    Bk = st.Btile + (gm.b_blk ? (int64_t)ks * gm.b_blk * kBK : k0);
  }
  uint8_t* stage = lds + (g % kStages) * C::STAGE_BYTES;
#pragma unroll
  for (int t = 0; t < C::PER_WAVE; ++t) {
    uint32_t off = st.off[t];
    if (KTAIL) {
      const int row = (cw + kCopyWaves * t) * 8 + (lane >> 3);
      const int kc = k0 + (((lane & 7) ^ swz_key(row)) << 4);
      if (kc >= gm.K) off -= (uint32_t)(kc - (gm.K - 16));
    }
#if defined(__HIP_DEVICE_COMPILE__)  // an AMDGPU builtin: the host pass never runs this
    __builtin_amdgcn_global_load_lds((t < C::A_PER_WAVE ? Ak : Bk) + off,
                                     stage + (cw + kCopyWaves * t) * 1024, 16, 0, 0);
#else
    (void)off;
    (void)stage;
    (void)Ak;
    (void)Bk;
#endif
  }
}

template <class C>
__device__ __forceinline__ void zero_tail(uint8_t* stage, int K, int ks, int cw, int lane) {
  const int k0 = ks * kBK;
  if (k0 + kBK <= K) return;
#pragma unroll
  for (int t = 0; t < C::PER_WAVE; ++t) {
    const int blk = cw + kCopyWaves * t;
    const int row = blk * 8 + (lane >> 3);
    const int kc = k0 + (((lane & 7) ^ swz_key(row)) << 4);
    if (kc >= K) *reinterpret_cast<uint4*>(stage + blk * 1024 + lane * 16) = make_uint4(0, 0, 0, 0);
  }
}

// Wait until step g has landed in its stage (every step after it that is
// already issued may stay in flight: at most one, of PER_WAVE loads).
template <class C, bool KTAIL>
__device__ __forceinline__ void land(const CopyState<C>& st, uint8_t* lds, const Gemm& gm,
                                     const Sched& sc, int g, int cw, int lane) {
  if (st.issued > g + 1)
    wait_vm<C::PER_WAVE>();
  else
    wait_vm<0>();
  if (KTAIL) zero_tail<C>(lds + (g % kStages) * C::STAGE_BYTES, gm.K, sc.ks(g), cw, lane);
}

// The copy waves' side of the pipeline.  Before barrier -1 steps 0 and 1
// are issued and step 0 has landed; in iteration g step g + 2 is issued
// into the stage step g - 1 used (read before barrier g - 1) and step g + 1
// has landed before barrier g.
template <class C, bool KTAIL>
__device__ __forceinline__ void copy_role(uint8_t* lds, const Gemm& gm, const Sched& sc, int cw,
                                          int lane) {
  CopyState<C> st;
  st.tile = -1;
  st.issued = 0;
  if (sc.steps > 0) issue_next<C, KTAIL>(st, lds, gm, sc, cw, lane);
  if (sc.steps > 1) issue_next<C, KTAIL>(st, lds, gm, sc, cw, lane);
  if (sc.steps > 0) land<C, KTAIL>(st, lds, gm, sc, 0, cw, lane);
  barrier_lds();
  for (int g = 0; g < sc.steps; ++g) {
    if (g + 2 < sc.steps) issue_next<C, KTAIL>(st, lds, gm, sc, cw, lane);
    if (g + 1 < sc.steps) land<C, KTAIL>(st, lds, gm, sc, g + 1, cw, lane);
    barrier_lds();
  }
}

// ------------------------------------------------------------ matrix waves

// Operand fragments of one K half-step (64 bytes of K) of a matrix wave.
template <class C>
struct Half {
  v8i a[C::FM];
  v8i b[C::FN];
};

template <class C, bool TOK>
__device__ __forceinline__ void load_half(const uint8_t* stage, int a0, int b0, int lane, int h,
                                          Half<C>& f) {
#pragma unroll
  for (int j = 0; j < C::FN; ++j) f.b[j] = frag_b<C, TOK>(stage, b0 + j * 32, lane, h);
#pragma unroll
  for (int i = 0; i < C::FM; ++i) f.a[i] = frag_a<C, TOK>(stage, a0 + i * 32, lane, h);
}

// The FM x FN MFMAs of one half-step on the operands in f, while the
// operands of the half-step after it (K half h of stage `src`) stream into
// f: its B fragments first, then A fragment i as soon as the current A
// fragment i has had its last use.  A fragment is thus loaded a whole
// half-step (FM x FN MFMAs) before it is needed.
// FIRST: the tile's first half-step, whose MFMAs start from zero rather
// than from acc.
template <class C, bool TOK, bool FIRST = false>
__device__ __forceinline__ void mma_half(v16f (&acc)[C::FM][C::FN], Half<C>& f, const uint8_t* src,
                                         int a0, int b0, int lane, int h) {
  v8i nb[C::FN];
#pragma unroll
  for (int j = 0; j < C::FN; ++j) nb[j] = frag_b<C, TOK>(src, b0 + j * 32, lane, h);
#pragma unroll
  for (int i = 0; i < C::FM; ++i) {
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc[i][j] = mfma32<C>(f.b[j], f.a[i], FIRST ? v16f{} : acc[i][j]);
    f.a[i] = frag_a<C, TOK>(src, a0 + i * 32, lane, h);
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, TOK ? 4 : 2, 0);  // then LDS reads
    }
  }
#pragma unroll
  for (int j = 0; j < C::FN; ++j) f.b[j] = nb[j];
}

// The second half-step of a step, around the step's barrier: its first
// kEarlyRows rows of MFMAs (whose operands streamed in early in the first
// half-step) go before the barrier, so that the barrier's wait for this
// wave's last LDS reads overlaps matrix work; the operands of half h of
// stage `src`, which the barrier releases, stream in behind the rest.
constexpr int kEarlyRows = 2;

template <class C, bool TOK>
__device__ __forceinline__ void mma_half_barrier(v16f (&acc)[C::FM][C::FN], Half<C>& f,
                                                 const uint8_t* src, int a0, int b0, int lane,
                                                 int h) {
  constexpr int ER = kEarlyRows < C::FM ? kEarlyRows : C::FM - 1;  // rows before the barrier
  static_assert(ER >= 1, "rows on both sides of the barrier");
#pragma unroll
  for (int i = 0; i < ER; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc[i][j] = mfma32<C>(f.b[j], f.a[i], acc[i][j]);
  // scheduling fences: the barrier orders memory accesses only, and the
  // compiler would otherwise sink the early MFMAs below it
  __builtin_amdgcn_sched_barrier(0);
  barrier_lds();
  __builtin_amdgcn_sched_barrier(0);
  v8i nb[C::FN];
#pragma unroll
  for (int j = 0; j < C::FN; ++j) nb[j] = frag_b<C, TOK>(src, b0 + j * 32, lane, h);
#pragma unroll
  for (int i = 0; i < ER; ++i) f.a[i] = frag_a<C, TOK>(src, a0 + i * 32, lane, h);
#pragma unroll
  for (int i = ER; i < C::FM; ++i) {
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc[i][j] = mfma32<C>(f.b[j], f.a[i], acc[i][j]);
    f.a[i] = frag_a<C, TOK>(src, a0 + i * 32, lane, h);
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, TOK ? 4 : 2, 0);  // then LDS reads
    }
  }
#pragma unroll
  for (int j = 0; j < C::FN; ++j) f.b[j] = nb[j];
}

// The same two steps with the loops the other way round, for wave tiles
// with more B than A fragments (FN > FM): the A fragments of the next
// half-step stream in first and B fragment j is reloaded after its last
// use, so that the fewer fragments are the ones held twice.
template <class C, bool TOK, bool FIRST = false>
__device__ __forceinline__ void mma_half_bo(v16f (&acc)[C::FM][C::FN], Half<C>& f,
                                            const uint8_t* src, int a0, int b0, int lane, int h) {
  v8i na[C::FM];
#pragma unroll
  for (int i = 0; i < C::FM; ++i) na[i] = frag_a<C, TOK>(src, a0 + i * 32, lane, h);
#pragma unroll
  for (int j = 0; j < C::FN; ++j) {
#pragma unroll
    for (int i = 0; i < C::FM; ++i) acc[i][j] = mfma32<C>(f.b[j], f.a[i], FIRST ? v16f{} : acc[i][j]);
    f.b[j] = frag_b<C, TOK>(src, b0 + j * 32, lane, h);
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, TOK ? 4 : 2, 0);  // then LDS reads
    }
  }
#pragma unroll
  for (int i = 0; i < C::FM; ++i) f.a[i] = na[i];
}

template <class C, bool TOK>
__device__ __forceinline__ void mma_half_barrier_bo(v16f (&acc)[C::FM][C::FN], Half<C>& f,
                                                    const uint8_t* src, int a0, int b0,
                                                    int lane, int h) {
  constexpr int EJ = kEarlyRows < C::FN ? kEarlyRows : C::FN - 1;  // columns before the barrier
  static_assert(EJ >= 1, "columns on both sides of the barrier");
#pragma unroll
  for (int j = 0; j < EJ; ++j)
#pragma unroll
    for (int i = 0; i < C::FM; ++i) acc[i][j] = mfma32<C>(f.b[j], f.a[i], acc[i][j]);
  __builtin_amdgcn_sched_barrier(0);
  barrier_lds();
  __builtin_amdgcn_sched_barrier(0);
  v8i na[C::FM];
#pragma unroll
  for (int i = 0; i < C::FM; ++i) na[i] = frag_a<C, TOK>(src, a0 + i * 32, lane, h);
#pragma unroll
  for (int j = 0; j < EJ; ++j) f.b[j] = frag_b<C, TOK>(src, b0 + j * 32, lane, h);
#pragma unroll
  for (int j = EJ; j < C::FN; ++j) {
#pragma unroll
    for (int i = 0; i < C::FM; ++i) acc[i][j] = mfma32<C>(f.b[j], f.a[i], acc[i][j]);
    f.b[j] = frag_b<C, TOK>(src, b0 + j * 32, lane, h);
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, TOK ? 4 : 2, 0);  // then LDS reads
    }
  }
#pragma unroll
  for (int i = 0; i < C::FM; ++i) f.a[i] = na[i];
}

template <class C>
__device__ __forceinline__ void zero_acc(v16f (&acc)[C::FM][C::FN]) {
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
}

// The matrix waves' pipeline over the block's steps.  Half 0 of step g
// was loaded after barrier g - 1; half 1 streams in during half 0's MFMAs;
// then (after the first rows of half 1's MFMAs) barrier g: all of this
// wave's reads of step g are done and step g + 1 has landed; half 0 of
// step g + 1 streams in during the rest of half 1's MFMAs.
// `tile_start()` runs before the first K step of each tile and
// `tile_done(acc)` after its last one (every nk steps).  With ZC the first half-step of every tile starts from zero
// accumulators and tile_done may leave acc as it is; without it tile_done
// must zero acc.  After the block's last step the stream reads a stage
// whose contents are not used.
template <class C, bool TOK, bool ZC, class TileDone, class TileStart>
__device__ __forceinline__ void mma_role(const uint8_t* lds, const Sched& sc, int wm, int wn,
                                         int lane, v16f (&acc)[C::FM][C::FN],
                                         const TileDone& tile_done, const TileStart& tile_start) {
  const int a0 = wm * C::WM, b0 = wn * C::WN;
  if (!ZC) zero_acc<C>(acc);
  barrier_lds();
  Half<C> f;
  load_half<C, TOK>(lds, a0, b0, lane, 0, f);
  // one K step: half 1 of the step's stage, then half 0 of the next one
  // around the step's barrier; FIRST starts the tile's accumulators from zero
  auto step = [&](int g, auto first) {
    constexpr bool FIRST = decltype(first)::value;
    const uint8_t* cur = lds + (g % kStages) * C::STAGE_BYTES;
    const uint8_t* nxt = lds + ((g + 1) % kStages) * C::STAGE_BYTES;
    if constexpr (C::FN > C::FM) {
      mma_half_bo<C, TOK, FIRST>(acc, f, cur, a0, b0, lane, 1);
      mma_half_barrier_bo<C, TOK>(acc, f, nxt, a0, b0, lane, 0);
    } else {
      mma_half<C, TOK, FIRST>(acc, f, cur, a0, b0, lane, 1);
      mma_half_barrier<C, TOK>(acc, f, nxt, a0, b0, lane, 0);
    }
  };
  // tile by tile, so that the accumulators are dead between a tile's
  // tile_done and the next tile's first step (with ZC, which writes them
  // from zero): the epilogue then has their registers
  for (int g = 0; g < sc.steps;) {
    tile_start();
    if (ZC)
      step(g, std::true_type{});
    else
      step(g, std::false_type{});
    ++g;
    for (int ks = 1; ks < sc.nk; ++ks, ++g) step(g, std::false_type{});
    tile_done(acc);
  }
}

// ------------------------------------------------------------ epilogues

// bf16 output chunks go out as streaming (non-temporal) stores: no wave of
// the kernel reads them back, and they would otherwise push the operand
// rows the other blocks are about to reuse out of L2.
typedef unsigned v4u __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_stream(uint16_t* p, uint4 v) {
  const v4u x = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(x, reinterpret_cast<v4u*>(p));
}

// An ordinary 16-byte store, for outputs whose cache lines are filled by
// several stores (from neighbouring rows or tiles) that the L2 must merge.
__device__ __forceinline__ void store_plain(uint16_t* p, uint4 v) {
  *reinterpret_cast<uint4*>(p) = v;
}

// bf16 tile store through the matrix wave's own LDS slice: 32 rows x WN
// columns (WN * 2 bytes per row, 16-byte chunks XOR-swizzled by row).  Each
// lane writes its 4-column groups, then reads back whole 16-byte chunks:
// lane l takes chunk l % 8 of rows l / 8 + 8q.  LDS operations of one wave
// complete in order, so no wait is needed between the two.
template <class C>
struct WaveSlice {
  static constexpr int BYTES = 32 * C::WN * 2;
  static_assert(C::WN == 64, "8 chunks of 16 bytes per row");
  __device__ static int at(int row, int chunk) {
    return row * (C::WN * 2) + ((chunk ^ (row & 7)) << 4);
  }
};

// Forward for head widths without the fused epilogue: Q|K columns to the
// pre-norm rows in the forward workspace (the norm/RoPE kernel reads them
// next), V columns straight into the head-major v output.  A chunk of 8 columns never straddles a V head
// (d_v % 16 == 0) nor the Q|K / V boundary.
struct EpiFwd {
  static constexpr bool kMap = false, kAux = false, kAmax = false;
  uint16_t* qk_pre;
  uint16_t* v;
  int N, nqk2, H, dv, S;
  struct Col { int n; int64_t voff; bool qk; bool live; };
  struct Row { int m; int b; int s; };
  __device__ Col column(int n) const {
    Col c{n, 0, n < nqk2, n < N};
    if (!c.qk && c.live) {
      const int nn = n - nqk2, h = nn / dv, j = nn - h * dv;
      c.voff = (int64_t)h * S * dv + j;
    }
    return c;
  }
  __device__ Row row(int m) const { return Row{m, m / S, m % S}; }
  __device__ void advance(Row& r, int step) const {
    r.m += step;
    r.s += step;
    while (r.s >= S) { r.s -= S; ++r.b; }
  }
  __device__ void chunk(const Row& r, const Col& c, uint4 val) const {
    if (!c.live) return;
    if (c.qk)
      store_stream(qk_pre + (int64_t)r.m * nqk2 + c.n, val);
    else
      store_stream(v + (int64_t)r.b * H * S * dv + (int64_t)r.s * dv + c.voff, val);
  }
  // Rows m0 .. m1 are rows of one sequence: each column's rows are then
  // evenly spaced in both outputs.
  __device__ bool one_run(int m0, int m1) const { return m0 / S == m1 / S; }
  __device__ uint16_t* at(int m, const Col& c) const {
    if (c.qk) return qk_pre + (int64_t)m * nqk2 + c.n;
    const int b = m / S, s = m - b * S;
    return v + (int64_t)b * H * S * dv + (int64_t)s * dv + c.voff;
  }
  __device__ int64_t step8(const Col& c) const { return 8 * (int64_t)(c.qk ? nqk2 : dv); }
};

// Plain [M][N] rows: dX of the QKV projection, and the MLP's y and dX.
struct EpiDx {
  static constexpr bool kMap = false, kAux = false, kAmax = false;
  uint16_t* dx;
  int N;
  struct Col { int n; bool live; };
  struct Row { int m; };
  __device__ Col column(int n) const { return Col{n, n < N}; }
  __device__ Row row(int m) const { return Row{m}; }
  __device__ void advance(Row& r, int step) const { r.m += step; }
  __device__ void chunk(const Row& r, const Col& c, uint4 val) const {
    if (c.live) store_stream(dx + (int64_t)r.m * N + c.n, val);
  }
  __device__ bool one_run(int, int) const { return true; }
  __device__ uint16_t* at(int m, const Col& c) const { return dx + (int64_t)m * N + c.n; }
  __device__ int64_t step8(const Col&) const { return 8 * (int64_t)N; }
};

// Epilogues that transform the product before it is rounded (map) also
// keep the largest |bf16| of what they store, per matrix wave, for the
// quantiser of their output: one partial per wave, slot block * 4 + wave,
// as the fp32 bit pattern of that bf16 value.
__device__ __forceinline__ void epi_partial(uint32_t* partials, uint32_t amax, int slot,
                                            int lane) {
  amax = wave_max_u32(amax);
  if (lane == 0) partials[slot] = amax << 16;
}

// The MLP's first projection, PR #344 page, "Changes" (the FP8 ReLU^2 MLP):
// h = relu(pre)^2 into [M][N] bf16 rows.  A NaN product stays NaN.
struct EpiRelu2 : EpiDx {
  static constexpr bool kMap = true, kAux = false, kAmax = true;
  uint32_t* partials;
  __device__ void prepare() {}
  __device__ void map(float (&v)[4], uint32_t) const {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float r = v[e] <= 0.0f ? 0.0f : v[e];
      v[e] = r * r;
    }
  }
  __device__ void finish(uint32_t amax, int slot, int lane) const {
    epi_partial(partials, amax, slot, lane);
  }
};

// The MLP's dh = dy W2^T turned into dpre = 2 dh relu(pre), with relu(pre)
// recovered as sqrt(s_h dec(h8)) from the kept h^2 codes (PR #344 page,
// "Changes": no pre-activation is kept), computed as dh sqrt(4 s_h
// dec(h8)) with the hardware square root (1 ulp; the result is rounded to
// bf16).  h8 is in the blocked
// row layout (kc blocks of kKBlock columns per block row); aux_row() points
// at the code of column n of row m, and the codes of a lane's columns n +
// 32 j + 8 g, which share that 128-column block, follow at fixed offsets.
struct EpiDpre : EpiDx {
  static constexpr bool kMap = true, kAux = true, kAmax = true;
  uint32_t* partials;
  const uint8_t* h8;
  const float* h_scales;
  int kc;
  float sh4;
  __device__ void prepare() { sh4 = 4.0f * h_scales[0]; }
  __device__ const uint8_t* aux_row(int m, int n) const {
    const int64_t blk = (int64_t)(m / kActRows) * kc + n / kKBlock;
    return h8 + (blk * kActRows + m % kActRows) * kKBlock + n % kKBlock;
  }
  __device__ void map(float (&v)[4], uint32_t codes) const {
    const v2f_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)codes, false);  // bytes 0, 1
    const v2f_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)codes, true);   // bytes 2, 3
    const float h[4] = {lo.x, lo.y, hi.x, hi.y};
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] *= __builtin_amdgcn_sqrtf(sh4 * h[e]);
  }
  __device__ void finish(uint32_t amax, int slot, int lane) const {
    epi_partial(partials, amax, slot, lane);
  }
};

__device__ __forceinline__ uint32_t absmax_bf16x2(uint32_t w) {
  const uint32_t lo = w & 0x7fffu, hi = (w >> 16) & 0x7fffu;
  return lo > hi ? lo : hi;
}

// Lane (rq, p) of a wave's part (rows mp.., columns np..): the 8 auxiliary
// bytes of chunk p of rows mp + 32 i + rq + 8 q, q < 4, so that 8 lanes
// cover one row's 64 bytes.
template <class C, class Epi>
__device__ __forceinline__ void aux_slice(const Epi& epi, int mp, int np, int i, int lane,
                                          uint2 (&dst)[4]) {
  if constexpr (Epi::kAux) {
    const uint8_t* ar = epi.aux_row(mp + i * 32 + (lane >> 3), np + 8 * (lane & 7));
#pragma unroll
    for (int q = 0; q < 4; ++q)  // rows rq + 8q lie in the same block of kActRows rows
      dst[q] = *reinterpret_cast<const uint2*>(ar + q * 8 * kKBlock);
  }
}

template <class C, class Epi>
__device__ __forceinline__ void store_bf16_tile(const v16f (&acc)[C::FM][C::FN], float alpha,
                                                uint8_t* slice, const Epi& epi, int M, int m0,
                                                int n0, int wm, int wn, int lane,
                                                uint32_t& amax, const uint2 (&aux0)[4],
                                                const uint2 (&aux1)[4]) {
  using W = WaveSlice<C>;
  const int p = lane & 7, rq = lane >> 3;
  const typename Epi::Col col = epi.column(n0 + wn * C::WN + 8 * p);
  // Lane rows are mp + rq + 8k, k < 16.  When the part lies inside M and
  // inside one sequence each lane walks one pointer by a fixed stride;
  // otherwise every row is placed on its own.
  const int mp = m0 + wm * C::WM;
  const bool fast = mp + C::WM <= M && epi.one_run(mp, mp + C::WM - 1);
  typename Epi::Row row = epi.row(mp + rq);
  uint16_t* ptr = fast && col.live ? epi.at(mp + rq, col) : nullptr;
  const int64_t step = epi.step8(col);
  // this lane's accumulator columns: nl + 32 j + 8 g + 0..3
  const int nl = n0 + wn * C::WN + 4 * (lane >> 5);
  // Auxiliary bytes (one per output element, blocked like h8) of slice i
  // (aux_slice) pass through the wave's LDS slice (rows 72 bytes apart: 18
  // words, so the 32 rows x 2 words of one read below fall in 64 distinct
  // banks) into the lanes that hold the matching accumulators.  Those of
  // slices 0 and 1 were fetched when the tile started (aux0, aux1); slice
  // i + 2's are fetched while slice i is worked on.
  // The store path is chosen once per part (fast is uniform over the
  // wave), so each variant is straight-line code; with an auxiliary input
  // the two copies would no longer fit the registers, and the choice is
  // made per store instead.  fast_c is std::true_type, std::false_type or
  // the runtime flag.
  auto body = [&](auto fast_c) {
    static_assert(C::WN == 64, "64 auxiliary bytes per row");
    uint2 raw[4], nxt[4];
    if constexpr (Epi::kAux)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        raw[q] = aux0[q];
        nxt[q] = aux1[q];
      }
    auto aux_word = [](int row, int w) { return row * 72 + 4 * w; };
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
      const int ml = mp + i * 32 + (lane & 31);  // this lane's accumulator row
      uint32_t aux[C::FN][4];
      if constexpr (Epi::kAux) {
        // the wave's LDS operations complete in order: the reads below finish
        // before the bf16 writes reuse the slice
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<uint2*>(slice + aux_word(rq + 8 * q, 2 * p)) = raw[q];
#pragma unroll
        for (int q = 0; q < 4; ++q) raw[q] = nxt[q];
        if (i + 2 < C::FM) aux_slice<C, Epi>(epi, mp, n0 + wn * C::WN, i + 2, lane, nxt);
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            aux[j][g] = *reinterpret_cast<const uint32_t*>(
                slice + aux_word(lane & 31, 8 * j + 2 * g + (lane >> 5)));
      }
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const v16f& a = acc[i][j];
          float v[4] = {a[4 * g] * alpha, a[4 * g + 1] * alpha, a[4 * g + 2] * alpha,
                        a[4 * g + 3] * alpha};
          if constexpr (Epi::kMap) epi.map(v, Epi::kAux ? aux[j][g] : 0u);
          const uint32_t w0 = cvt_bf16x2_rn(v[0], v[1]), w1 = cvt_bf16x2_rn(v[2], v[3]);
          if constexpr (Epi::kAmax) {
            if (ml < M && nl + 32 * j + 8 * g < epi.N) {
              const uint32_t a01 = absmax_bf16x2(w0), a23 = absmax_bf16x2(w1);
              amax = max(amax, max(a01, a23));
            }
          }
          *reinterpret_cast<uint2*>(slice + W::at(lane & 31, 4 * j + g) + 8 * (lane >> 5)) =
              make_uint2(w0, w1);
        }
      uint4 val[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) val[q] = *reinterpret_cast<const uint4*>(slice + W::at(rq + 8 * q, p));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (static_cast<bool>(fast_c)) {
          if (col.live) store_stream(ptr, val[q]);
          ptr += step;
        } else {
          if (row.m < M) epi.chunk(row, col, val[q]);
          epi.advance(row, 8);
        }
      }
    }
  };
  if constexpr (Epi::kAux)
    body(fast);
  else if (fast)
    body(std::true_type{});
  else
    body(std::false_type{});
}

// fp32 split-K partials: lane l holds four consecutive n of one m.
template <class C>
__device__ __forceinline__ void store_partial_tile(const v16f (&acc)[C::FM][C::FN], float* part,
                                                   int M, int N, int m0, int n0, int wm, int wn,
                                                   int lane) {
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int m = m0 + wm * C::WM + i * 32 + (lane & 31);
        const int n = n0 + wn * C::WN + j * 32 + 8 * g + 4 * (lane >> 5);
        if (m < M && n < N)
          *reinterpret_cast<float4*>(part + (int64_t)m * N + n) =
              make_float4(acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                          acc[i][j][4 * g + 3]);
      }
}

// -------------------------------------------------- persistent bf16 GEMM

// Block b's tiles: per-XCD row panels when every XCD gets the same number
// of them, else simply tiles b, b + G, b + 2G, ...
__device__ __forceinline__ void persistent_tiles(Sched& sc, int b, int G, int ntiles,
                                                 int n_tiles) {
  const int m_tiles = ntiles / n_tiles;
  sc.single = -1;
  sc.n_tiles = n_tiles;
  if (G % 8 == 0 && m_tiles % 8 == 0) {
    sc.P = 8; sc.x = b % 8; sc.i = b / 8; sc.c = G / 8;
  } else {
    sc.P = 1; sc.x = 0; sc.i = b; sc.c = G;
  }
  const int total = (m_tiles - sc.x + sc.P - 1) / sc.P * n_tiles;
  const int mine = sc.i < total ? (total - sc.i + sc.c - 1) / sc.c : 0;
  sc.steps = mine * sc.nk;
}

// --------------------------------- forward with RMSNorm and RoPE fused in
//
// "96 is enough", "The change": after the one packed matmul, q and k are
// RMS-normalised and rotated; PR #344 page, "Changes": norm, RoPE and the
// layout conversion are fused.  Here they run in the matmul's own epilogue,
// so no pre-norm row ever reaches memory.  The tile is the bf16 GEMM's
// 256 x 128, its B rows fetched in head-aligned order (ColMap), and its
// four matrix waves each take 64 rows x all 128 columns: every Q/K head row
// of a tile lies inside one wave.  For row l % 32 (+ 32 i) a lane holds the
// tile's columns 8 g + 4 (l / 32) + e (g < 16, e < 4): a head row's sum of
// squares is the lane's own values plus one exchange with lane l ^ 32, and
// the rotation partner of head column c < d/2, c + d/2, sits in the same
// lane (group g + d/16, same e).  The product is rounded to bf16 first,
// exactly where an unfused path would store it, then normalised (fp32) and
// rotated; 1 / rms of every Q and K head row goes out with q, k and v, and
// the backward rebuilds the normalised rows from q and k with it.
// Stores: the 64-byte V pieces of a mixed tile fill a V row's cache lines
// only together with the neighbouring tiles' (same row panel, same XCD),
// so they are ordinary stores, which the L2 merges; everything else is
// streamed.  (Measured on the forward GEMM at 65536 tokens, fetched +
// written: all streamed 63 + 315 MB, this 65 + 302 MB, all ordinary 130 +
// 256 MB, the L2 then reading lines in before partial writes; the same
// time each.  The q / k rows, d * 2 bytes, fill whole lines only across
// the two 64-column passes.)

struct QkvOut {
  uint16_t* q;   // [n_seq][H][S][qs]
  uint16_t* k;
  uint16_t* v;   // [n_seq][H][S][dv]
  float* rho;    // [2][n_seq][H][S]: 1 / rms of each q row, then of each k row
  int H, S, dv, qs, n_seq;
  float eps;
};

// The rotation frequencies of a lane's head columns c = 8 idx + 4 (l / 32) +
// e, in revolutions per position: theta_c / (2 pi) = rev0 * r^(c - c0) with
// r = base^(-2/d).  A row's angles p theta_c / (2 pi) are stepped by one
// fp64 multiplication per column: with positions below 2^24 the angles
// stay below 2^22 revolutions, and over the at most 32 steps of a head
// their fractional parts keep an error below ~1e-8 revolutions before the
// fp32 sine.
struct RopeRev {
  double rev0;    // theta_c0 / (2 pi) of the lane's first column c0 = 4 (l / 32)
  double r1, r5;  // r and r^5: one column on, and from e = 3 to the next group
};

// 32 rows x 64 bf16 columns of a wave's LDS slice: row pitch 128 bytes,
// 16-byte chunks XOR-swizzled by row.
__device__ __forceinline__ int slice64(int row, int chunk) {
  return row * 128 + ((chunk ^ (row & 7)) << 4);
}

template <class C, int D>
__device__ __forceinline__ void store_qkv_tile(const v16f (&acc)[C::FM][C::FN], float alpha,
                                               uint8_t* slice, const RopeRev& rr,
                                               const QkvOut& o, const ColMap& cm, int M, int m0,
                                               int nt, int wm, int lane) {
  constexpr int HPT = 128 / D, G = D / 8, HG = G / 2, VG0 = HPT * G;  // V groups from VG0 on
  static_assert(C::WN == 128 && C::FN == 4 && C::WM == 64, "whole tile rows per matrix wave");
  const bool mixed = nt < cm.n_mixed;
  const int r = lane & 31, hl = lane >> 5;
  const int mp = m0 + wm * C::WM;
  // the part's rows lie inside M and one sequence: rows follow each other
  // in every output (else each row is placed on its own)
  const int b0 = mp / o.S, s0 = mp - b0 * o.S;
  const bool fast = mp + C::WM <= M && (mp + C::WM - 1) / o.S == b0;
  // element offset of token m's row in head hh of an [n_seq][H][S][w] output
  auto row_off = [&](int m, int hh, int w) -> int64_t {
    int b = b0, sp = s0 + (m - mp);
    if (!fast) { b = m / o.S; sp = m - b * o.S; }
    return (((int64_t)b * o.H + hh) * o.S + sp) * w;
  };
  const int hq0 = nt * HPT;  // the tile's first packed head (Q heads, then K heads)
  auto head_ok = [&](int hs) { return mixed && hq0 + hs < 2 * o.H; };
  // the whole product of the part, rounded to bf16 (packed pairs), first:
  // the fp32 accumulators die here, which leaves room for the norm and
  // rotation (the opaque step keeps the compiler from sinking the
  // conversions back to their uses)
  uint2 P[C::FM][16];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int g = 0; g < 16; ++g) {
      const v16f& a = acc[i][g / 4];
      const int q4 = g % 4;
      P[i][g] = make_uint2(cvt_bf16x2_rn(a[4 * q4] * alpha, a[4 * q4 + 1] * alpha),
                           cvt_bf16x2_rn(a[4 * q4 + 2] * alpha, a[4 * q4 + 3] * alpha));
      asm volatile("" : "+v"(P[i][g].x), "+v"(P[i][g].y));
    }
  // The output of tile group g (8 columns): a Q/K head's row (array, head,
  // row width, first column), or a V head's row, or none.  V column f's
  // head f / d_v comes from a float product: f < H d_v <= 2^16, so
  // (f + 0.5) / d_v is off by far less than 0.5 / d_v.
  struct Dst {
    uint16_t* arr;
    int hh, w, col;
  };
  const float inv_dv = 1.0f / (float)o.dv;
  auto chunk_dst = [&](int g) -> Dst {
    Dst d{nullptr, 0, 0, 0};
    if (mixed && g < VG0) {
      const int hs = g / G;
      if (head_ok(hs)) {
        const int hq = hq0 + hs;
        const bool isk = hq >= o.H;
        d = Dst{isk ? o.k : o.q, isk ? hq - o.H : hq, o.qs, 8 * (g - hs * G)};
      }
    } else {  // the filler of a mixed tile, or a whole-V tile
      const int f = mixed ? nt * cm.fill + 8 * (g - VG0)
                          : cm.n_mixed * cm.fill + (nt - cm.n_mixed) * 128 + 8 * g;
      if (f < cm.nv) {
        const int hh = (int)(((float)f + 0.5f) * inv_dv);
        d = Dst{o.v, hh, o.dv, f - hh * o.dv};
      }
    }
    return d;
  };
  // fast path: where lane (rq, pc)'s chunk of pass ps goes for row mp + rq
  // (fragment i adds 32 i rows), once per tile
  const int pc = lane & 7, rq = lane >> 3;
  uint16_t* fdst[2] = {nullptr, nullptr};
  int fw[2] = {0, 0};
  if (fast) {
#pragma unroll
    for (int ps = 0; ps < 2; ++ps) {
      const Dst d = chunk_dst(8 * ps + pc);
      if (d.arr) fdst[ps] = d.arr + (((int64_t)(b0 * o.H + d.hh) * o.S + s0 + rq) * d.w + d.col);
      fw[ps] = d.w;
    }
  }
  auto unpack4 = [](uint2 w, float (&f)[4]) {
    f[0] = __uint_as_float(w.x << 16);
    f[1] = __uint_as_float(w.x & 0xffff0000u);
    f[2] = __uint_as_float(w.y << 16);
    f[3] = __uint_as_float(w.y & 0xffff0000u);
  };
  // Norm and rotation of both fragments first, in place in P (the two
  // fragments' chains are independent, which gives the scheduler work to
  // overlap); then the stores.
#pragma unroll
  for (int i = 0; i < C::FM; ++i) {
    if (!mixed) break;  // uniform: a tile of V columns only
    const int m = mp + 32 * i + r;  // this lane's row
    int b = b0, p = s0 + 32 * i + r;  // its sequence and position
    if (!fast) {
      b = m / o.S;
      p = m - b * o.S;
    }
#pragma unroll
    for (int hs = 0; hs < HPT; ++hs) {
      if (!head_ok(hs)) continue;  // uniform
      float ss = 0.f;  // the row's sum of squares, bf16 pairs at a time
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const uint2 w = P[i][hs * G + g];
        ss = dot2_bf16(w.y, w.y, dot2_bf16(w.x, w.x, ss));
      }
      {  // plus the other half of the row, in lane l ^ 32 (same sum on both)
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(ss),
                                                         __float_as_uint(ss), false, false);
        ss = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      }
      const float rho = 1.0f / sqrtf(ss / (float)D + o.eps);
      if (hl == 0 && m < M) {
        const bool isk = hq0 + hs >= o.H;
        const int hh = isk ? hq0 + hs - o.H : hq0 + hs;
        // [2][n_seq][H][S]: row (isk, b, hh, p)
        o.rho[((int64_t)(isk * o.n_seq + b) * o.H + hh) * o.S + p] = rho;
      }
      // the pairs (idx, idx + d/16), rotated in place; the row's angle in
      // revolutions, p theta_c / (2 pi), is stepped from column to column
      // like the frequency (opaque to the compiler: the chain is formed here,
      // per tile, instead of being hoisted out of the tile loop, where its
      // doubles would stay live through the matrix work)
      double ang = rr.rev0;
      asm volatile("" : "+v"(ang));
      ang *= (double)p;
#pragma unroll
      for (int idx = 0; idx < HG; ++idx) {
        const int glo = hs * G + idx, ghi = glo + HG;
        float y1[4], y2[4], o1[4], o2[4];
        unpack4(P[i][glo], y1);
        unpack4(P[i][ghi], y2);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float f = (float)__builtin_amdgcn_fract(ang);  // in [0, 1)
          const float sn = __builtin_amdgcn_sinf(f);          // sin(2 pi f)
          const float cn = __builtin_amdgcn_cosf(f);
          ang *= e < 3 ? rr.r1 : rr.r5;
          const float u1 = y1[e] * rho, u2 = y2[e] * rho;
          o1[e] = u1 * cn - u2 * sn;
          o2[e] = u2 * cn + u1 * sn;
        }
        P[i][glo] = make_uint2(cvt_bf16x2_rn(o1[0], o1[1]), cvt_bf16x2_rn(o1[2], o1[3]));
        P[i][ghi] = make_uint2(cvt_bf16x2_rn(o2[0], o2[1]), cvt_bf16x2_rn(o2[2], o2[3]));
      }
    }
  }
#pragma unroll
  for (int i = 0; i < C::FM; ++i) {
    // two passes of 64 columns: lane (rq, pc) stores chunk pc of rows
    // rq + 8 q, q < 4 (8 rows x 128 bytes per store instruction)
#pragma unroll
    for (int ps = 0; ps < 2; ++ps) {
#pragma unroll
      for (int g = 8 * ps; g < 8 * ps + 8; ++g)
        *reinterpret_cast<uint2*>(slice + slice64(r, g & 7) + 8 * hl) = P[i][g];
      uint4 val[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        val[q] = *reinterpret_cast<const uint4*>(slice + slice64(rq + 8 * q, pc));
      if (fast) {  // rows rq + 8 q follow each other: one pointer, fixed stride
        if (fdst[ps]) {
          uint16_t* at = fdst[ps] + 32 * i * fw[ps];
          if (mixed && 8 * ps + pc >= VG0) {  // a 64-byte piece of a V row
#pragma unroll
            for (int q = 0; q < 4; ++q, at += 8 * fw[ps]) store_plain(at, val[q]);
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q, at += 8 * fw[ps]) store_stream(at, val[q]);
          }
        }
      } else {
        const Dst d = chunk_dst(8 * ps + pc);
        if (d.arr) {
          const int mt0 = mp + 32 * i + rq;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int mt = mt0 + 8 * q;
            if (mt < M) store_stream(d.arr + row_off(mt, d.hh, d.w) + d.col, val[q]);
          }
        }
      }
    }
    // zero padding columns d .. qs - 1 of the fragment's q / k rows
    if (o.qs > D) {
      const int pcs = (o.qs - D) / 8;
#pragma unroll
      for (int hs = 0; hs < HPT; ++hs) {
        if (!head_ok(hs)) continue;
        const int hq = hq0 + hs;
        const bool isk = hq >= o.H;
        for (int it = lane; it < 32 * pcs; it += 64) {
          const int rw = it / pcs, c = it - rw * pcs;
          const int mt = mp + 32 * i + rw;
          if (mt < M)
            store_stream((isk ? o.k : o.q) + row_off(mt, isk ? hq - o.H : hq, o.qs) + D + 8 * c,
                         make_uint4(0, 0, 0, 0));
        }
      }
    }
  }
}

template <int D, bool KTAIL>
__global__ __launch_bounds__((TileCfg<256, 128, 4, 1>::THREADS), 1) void gemm_qkv_fwd_kernel(
    Gemm gm, int ntiles, const float* __restrict__ sa, const float* __restrict__ sb, QkvOut o,
    float base) {
  using C = TileCfg<256, 128, 4, 1>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kStages * C::STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t slices[C::MMA * 4096];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  Sched sc;
  sc.nk = (gm.K + kBK - 1) / kBK;
  sc.ks0 = 0;
  persistent_tiles(sc, blockIdx.x, gridDim.x, ntiles, gm.n_tiles);
  if (wave >= C::MMA) {
    copy_role<C, KTAIL>(lds, gm, sc, wave - C::MMA, lane);
    return;
  }
  const float alpha = sa[0] * sb[0];
  uint8_t* slice = slices + wave * 4096;
  const double r1 = rope_rev(1, D, base) / rope_rev(0, D, base);
  const RopeRev rr{rope_rev(4 * (lane >> 5), D, base), r1, r1 * r1 * r1 * r1 * r1};
  int ord = 0;
  v16f acc[C::FM][C::FN];
  auto done = [&](v16f (&a)[C::FM][C::FN]) {
    const int tile = sc.tile_of(ord++);
    store_qkv_tile<C, D>(a, alpha, slice, rr, o, gm.cm, gm.M, (tile / gm.n_tiles) * C::BM_,
                         tile % gm.n_tiles, wave, lane);
  };
  mma_role<C, false, true>(lds, sc, wave, 0, lane, acc, done, [] {});
}

template <int BM, int BN, bool KTAIL, class Epi, int FA = kFmtE4M3>
__global__ __launch_bounds__((TileCfg<BM, BN>::THREADS), 1) void gemm_bf16out_kernel(
    Gemm gm, int ntiles, const float* __restrict__ sa, const float* __restrict__ sb, Epi epi) {
  using C = TileCfg<BM, BN, 2, 2, FA>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kStages * C::STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t slices[C::MMA * WaveSlice<C>::BYTES];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = gridDim.x;
  Sched sc;
  sc.nk = (gm.K + kBK - 1) / kBK;
  sc.ks0 = 0;
  persistent_tiles(sc, blockIdx.x, G, ntiles, gm.n_tiles);
  if (wave >= C::MMA) {
    copy_role<C, KTAIL>(lds, gm, sc, wave - C::MMA, lane);
    return;
  }
  const int wm = wave / C::NW_, wn = wave % C::NW_;
  const float alpha = sa[0] * sb[0];
  uint8_t* slice = slices + wave * WaveSlice<C>::BYTES;
  int ord = 0;
  uint32_t amax = 0;
  Epi e = epi;
  if constexpr (Epi::kMap) e.prepare();
  v16f acc[C::FM][C::FN];
  // an epilogue's auxiliary bytes for the tile's first two 32-row slices
  // are fetched when the tile starts, so that they arrive during its K steps
  uint2 aux0[4], aux1[4];
  auto start = [&] {
    if constexpr (Epi::kAux) {
      const int tile = sc.tile_of(ord);
      aux_slice<C, Epi>(e, (tile / gm.n_tiles) * BM + wm * C::WM,
                        (tile % gm.n_tiles) * BN + wn * C::WN, 0, lane, aux0);
      aux_slice<C, Epi>(e, (tile / gm.n_tiles) * BM + wm * C::WM,
                        (tile % gm.n_tiles) * BN + wn * C::WN, 1, lane, aux1);
    }
  };
  mma_role<C, false, true>(
      lds, sc, wm, wn, lane, acc,
      [&](v16f (&a)[C::FM][C::FN]) {
        const int tile = sc.tile_of(ord++);
        store_bf16_tile<C, Epi>(a, alpha, slice, e, gm.M, (tile / gm.n_tiles) * BM,
                                (tile % gm.n_tiles) * BN, wm, wn, lane, amax, aux0, aux1);
      },
      start);
  if constexpr (Epi::kAmax) e.finish(amax, blockIdx.x * C::MMA + wave, lane);
}

// ------------------------------------------------------------ dW split-K

// The (split, tile) items in that order, tile = m * n_tiles + n, are dealt
// to the XCDs in contiguous runs (blocks go round-robin over the 8 XCDs),
// so the blocks of one XCD share K ranges and rows of both operands in its
// L2.  Unscaled fp32 partial sums go to part[split][m][n]; a split with no
// K steps writes zeros.
template <int BM, int BN, int MW, int NW, int FB = kFmtE4M3>
__global__ __launch_bounds__((TileCfg<BM, BN, MW, NW>::THREADS), 1) void gemm_dw_part_kernel(
    Gemm gm, int splits, int ksteps_per_split, float* __restrict__ part) {
  using C = TileCfg<BM, BN, MW, NW, kFmtE4M3, FB>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kStages * C::STAGE_BYTES];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = gridDim.x, b = blockIdx.x, tiles = G / splits;
  // blocks go round-robin over the 8 XCDs: XCD x holds blocks x, x + 8, ...
  // and takes the items from x * (G / 8) + min(x, G % 8) on, in order
  const int x = b % 8, item = x * (G / 8) + min(x, G % 8) + b / 8;
  const int split = item / tiles, tile = item - split * tiles;
  const int nk_all = (gm.K + kBK - 1) / kBK;
  Sched sc;
  sc.ks0 = split * ksteps_per_split;
  sc.steps = max(0, min(nk_all, sc.ks0 + ksteps_per_split) - sc.ks0);
  sc.nk = sc.steps > 0 ? sc.steps : 1;
  sc.single = tile;
  if (wave >= C::MMA) {
    copy_role<C, false>(lds, gm, sc, wave - C::MMA, lane);
    return;
  }
  const int wm = wave / C::NW_, wn = wave % C::NW_;
  v16f acc[C::FM][C::FN];
  mma_role<C, true, false>(lds, sc, wm, wn, lane, acc, [](v16f (&)[C::FM][C::FN]) {}, [] {});
  store_partial_tile<C>(acc, part + (int64_t)split * gm.M * gm.N, gm.M, gm.N,
                        (tile / gm.n_tiles) * BM, (tile % gm.n_tiles) * BN, wm, wn, lane);
}

// Sum the split-K partials in split order (deterministic), scale, and write
// the three column blocks of dW.  Block (x, y) covers float4s
// 256 x .. 256 x + 255 of rows y, y + gridDim.y, ...
__global__ __launch_bounds__(kThreads) void dw_reduce_kernel(
    const float* __restrict__ part, int splits, int D, int N, const float* __restrict__ sx,
    const float* __restrict__ sg, int nq, float* __restrict__ dwq, int64_t ldq,
    float* __restrict__ dwk, int64_t ldk, float* __restrict__ dwv, int64_t ldv) {
  const int n = 4 * (blockIdx.x * kThreads + threadIdx.x);
  if (n >= N) return;
  const int64_t plane = (int64_t)D * N;
  const float alpha = sx[0] * sg[0];
  for (int d = blockIdx.y; d < D; d += gridDim.y) {
    const float* src = part + (int64_t)d * N + n;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k = 0; k < splits; ++k) {
      const float4 p = *reinterpret_cast<const float4*>(src + k * plane);
      s.x += p.x; s.y += p.y; s.z += p.z; s.w += p.w;
    }
    s = make_float4(s.x * alpha, s.y * alpha, s.z * alpha, s.w * alpha);
    float* dst = n < nq ? dwq + d * ldq + n : n < 2 * nq ? dwk + d * ldk + (n - nq)
                                                         : dwv + d * ldv + (n - 2 * nq);
    *reinterpret_cast<float4*>(dst) = s;
  }
}

// ------------------------------------------------------------- launchers

constexpr int kBMo = 256, kBNo = 128;  // bf16-output tile (persistent)
// dW split-K tile (token-major operands), 2 x 2 matrix waves of 128 x 64
// (4 x 2 waves of 64 x 64, two per SIMD, measured the same)
constexpr int kBMw = 256, kBNw = 128, kMWw = 2, kNWw = 2;
// Split-K counts are chosen for a 256-CU part; the choice must not depend on
// the device present, since workspace sizes are queried without one.
constexpr int kSplitCUs = 256, kMaxSplits = 8;
static_assert(kActRows == 2 * kBK, "a dW step is one half of a token block");

static int cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  return n;
}

// Returns the block count (the amax partial slots an epilogue with kAmax
// fills are blocks * 4, at most kEpiAmaxBlocks * 4).
constexpr int kEpiAmaxBlocks = 256;

template <class Epi, int FA = kFmtE4M3>
static int launch_bf16out(const Gemm& gm, const float* sa, const float* sb, const Epi& epi,
                          hipStream_t s) {
  const int ntiles = (int)ceil_div(gm.M, kBMo) * gm.n_tiles;
  const int cus = Epi::kAmax ? std::min(cu_count(), kEpiAmaxBlocks) : cu_count();
  const int blocks = ntiles < cus ? ntiles : cus;
  constexpr int kThr = TileCfg<kBMo, kBNo>::THREADS;
  if (gm.K % kBK)
    gemm_bf16out_kernel<kBMo, kBNo, true, Epi, FA><<<blocks, kThr, 0, s>>>(gm, ntiles, sa, sb, epi);
  else
    gemm_bf16out_kernel<kBMo, kBNo, false, Epi, FA><<<blocks, kThr, 0, s>>>(gm, ntiles, sa, sb, epi);
  return blocks;
}

int gemm_amax_slots_max() { return kEpiAmaxBlocks * TileCfg<kBMo, kBNo>::MMA; }

static_assert(kBMo == kActRows && kBK == kKBlock,
              "GEMM tiles and the blocked activation layouts");

void launch_gemm_fwd(const uint8_t* x8, const uint8_t* w_packed_t, int T, int N, int D,
                     const float* x_scales, const float* w_scales, uint16_t* qk_pre, int nqk2,
                     uint16_t* v, int H, int d_v, int seq_len, hipStream_t s) {
  const Gemm gm{x8, 0, w_packed_t, D, T, N, D, (int)ceil_div(N, kBNo), kActRows, 0, 0};
  launch_bf16out(gm, x_scales, w_scales, EpiFwd{qk_pre, v, N, nqk2, H, d_v, seq_len}, s);
}

// The head-aligned tile order of the forward projection (ColMap).
static ColMap fwd_colmap(int H, int d_qk, int d_v) {
  ColMap cm{};
  cm.d = d_qk;
  cm.hpt = 128 / d_qk;
  cm.fill = 128 - cm.hpt * d_qk;
  cm.n_mixed = (int)ceil_div(2 * H, cm.hpt);
  cm.nqk2 = 2 * H * d_qk;
  cm.nv = H * d_v;
  return cm;
}

static int fwd_col_tiles(const ColMap& cm) {
  const int rest = cm.nv - cm.n_mixed * cm.fill;
  return cm.n_mixed + (rest > 0 ? (int)ceil_div(rest, 128) : 0);
}

// Head widths with the fused forward; the B offsets of its mapped rows are
// 32-bit, so the packed weight must stay under 2 GiB.
bool fused_forward(int d_qk, int64_t N, int D) {
  return (d_qk == 64 || d_qk == 96 || d_qk == 128) && N * D < ((int64_t)1 << 31);
}

template <int DQK>
static void launch_qkv_fwd_t(const Gemm& gm, int ntiles, const float* sa, const float* sb,
                             const QkvOut& o, float base, hipStream_t s) {
  constexpr int kThr = TileCfg<256, 128, 4, 1>::THREADS;
  const int blocks = std::min(ntiles, cu_count());
  if (gm.K % kBK)
    gemm_qkv_fwd_kernel<DQK, true><<<blocks, kThr, 0, s>>>(gm, ntiles, sa, sb, o, base);
  else
    gemm_qkv_fwd_kernel<DQK, false><<<blocks, kThr, 0, s>>>(gm, ntiles, sa, sb, o, base);
}

void launch_gemm_qkv_fwd(const uint8_t* x8, const uint8_t* w_packed_t, int n_seq, int seq_len,
                         int D, int H, int d_qk, int d_v, int qs, float eps, float base,
                         const float* x_scales, const float* w_scales, uint16_t* q, uint16_t* k,
                         uint16_t* v, float* rho, hipStream_t s) {
  const int T = n_seq * seq_len, N = 2 * H * d_qk + H * d_v;
  const ColMap cm = fwd_colmap(H, d_qk, d_v);
  Gemm gm{x8, 0, w_packed_t, D, T, N, D, fwd_col_tiles(cm), kActRows, 0, 0};
  gm.cm = cm;
  const int ntiles = (int)ceil_div(T, kBMo) * gm.n_tiles;
  const QkvOut o{q, k, v, rho, H, seq_len, d_v, qs, n_seq, eps};
  switch (d_qk) {
    case 64: launch_qkv_fwd_t<64>(gm, ntiles, x_scales, w_scales, o, base, s); break;
    case 96: launch_qkv_fwd_t<96>(gm, ntiles, x_scales, w_scales, o, base, s); break;
    case 128: launch_qkv_fwd_t<128>(gm, ntiles, x_scales, w_scales, o, base, s); break;
    default: break;
  }
}

void launch_gemm_dx(const uint8_t* g8, const uint8_t* w_packed, int T, int D, int Np,
                    const float* g_scales, const float* w_scales, uint16_t* dx, hipStream_t s,
                    bool g_e5m2) {
  const Gemm gm{g8, 0, w_packed, Np, T, D, Np, (int)ceil_div(D, kBNo), kActRows, 0, 0};
  if (g_e5m2)
    launch_bf16out<EpiDx, kFmtE5M2>(gm, g_scales, w_scales, EpiDx{dx, D}, s);
  else
    launch_bf16out(gm, g_scales, w_scales, EpiDx{dx, D}, s);
}

int launch_gemm_relu2(const uint8_t* x8, const uint8_t* w1_t, int T, int F, int D,
                      const float* x_scales, const float* w_scales, uint16_t* h,
                      uint32_t* partials, hipStream_t s) {
  const Gemm gm{x8, 0, w1_t, D, T, F, D, (int)ceil_div(F, kBNo), kActRows, 0, 0};
  EpiRelu2 epi{};
  epi.dx = h;
  epi.N = F;
  epi.partials = partials;
  return launch_bf16out(gm, x_scales, w_scales, epi, s) * TileCfg<kBMo, kBNo>::MMA;
}

int launch_gemm_dpre(const uint8_t* dy8, const uint8_t* w2, int T, int F, int D,
                     const float* dy_scales, const float* w_scales, const uint8_t* h8,
                     const float* h_scales, uint16_t* dpre, uint32_t* partials, hipStream_t s,
                     bool dy_e5m2) {
  const Gemm gm{dy8, 0, w2, D, T, F, D, (int)ceil_div(F, kBNo), kActRows, 0, 0};
  EpiDpre epi{};
  epi.dx = dpre;
  epi.N = F;
  epi.partials = partials;
  epi.h8 = h8;
  epi.h_scales = h_scales;
  epi.kc = (int)ceil_div(F, kKBlock);
  const int blocks = dy_e5m2 ? launch_bf16out<EpiDpre, kFmtE5M2>(gm, dy_scales, w_scales, epi, s)
                             : launch_bf16out(gm, dy_scales, w_scales, epi, s);
  return blocks * TileCfg<kBMo, kBNo>::MMA;
}

// The split count s <= kMaxSplits (and <= the K steps) whose tiles x s
// blocks fill the last round of kSplitCUs best; ties go to fewer splits.
int dw_splits(int D, int Np, int64_t tokens_padded) {
  const int64_t nk = ceil_div(tokens_padded, kBK);
  const int64_t tiles = ceil_div(D, kBMw) * ceil_div(Np, kBNw);
  int best = 1;
  double best_fill = 0.0;
  for (int sp = 1; sp <= kMaxSplits && sp <= nk; ++sp) {
    const int64_t blocks = tiles * sp;
    const double fill = (double)blocks / (double)(ceil_div(blocks, kSplitCUs) * kSplitCUs);
    if (fill > best_fill + 1e-9) { best_fill = fill; best = sp; }
  }
  return best;
}

size_t dw_partial_bytes(int D, int Np, int64_t tokens_padded) {
  return (size_t)dw_splits(D, Np, tokens_padded) * D * Np * sizeof(float);
}

void launch_gemm_dw(const uint8_t* x8, const uint8_t* g8, int D, int Np, int64_t Tp,
                    float* part, hipStream_t s, bool g_e5m2) {
  const int splits = dw_splits(D, Np, Tp);
  const int nk = (int)ceil_div(Tp, kBK);
  const int per = (int)ceil_div(nk, splits);
  const Gemm gm{x8, ceil_div(D, kKBlock), g8, ceil_div(Np, kKBlock), D, Np, (int)Tp,
                (int)ceil_div(Np, kBNw), 0, 0, 1};
  const int blocks = (int)ceil_div(D, kBMw) * gm.n_tiles * splits;
  constexpr int kThr = TileCfg<kBMw, kBNw, kMWw, kNWw>::THREADS;
  if (g_e5m2)
    gemm_dw_part_kernel<kBMw, kBNw, kMWw, kNWw, kFmtE5M2><<<blocks, kThr, 0, s>>>(gm, splits, per,
                                                                                   part);
  else
    gemm_dw_part_kernel<kBMw, kBNw, kMWw, kNWw><<<blocks, kThr, 0, s>>>(gm, splits, per, part);
}

void launch_dw_reduce(const float* part, int D, int Np, int64_t Tp, const float* x_scales,
                      const float* g_scales, float* dwq, int64_t ldq, float* dwk, int64_t ldk,
                      float* dwv, int64_t ldv, int nq, hipStream_t s) {
  const dim3 grid((unsigned)ceil_div(Np / 4, kThreads), (unsigned)std::min(D, 32768));
  dw_reduce_kernel<<<grid, kThreads, 0, s>>>(part, dw_splits(D, Np, Tp), D, Np, x_scales,
                                             g_scales, nq, dwq, ldq, dwk, ldk, dwv, ldv);
}

}  // namespace fpr
