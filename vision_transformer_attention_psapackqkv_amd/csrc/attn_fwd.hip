// Flash Attention 2 forward for gfx950, and the fused PSA forward.
//
// vision-rs book, "Custom Kernels", section "Flash Attention 2": online
// softmax over [BATCH*N_HEADS, N_CTX, HEAD_DIM] tensors; the N_q x N_k score
// matrix is never stored. Section "Position-Sensitive Attention (PSA)": PSA
// runs FA2 once per V half (V_lo, V_hi) with HEAD_DIM = KEY_DIM, sharing Q and
// K. Since softmax(scale QK^T) does not depend on V, the fused kernel computes
// it once and multiplies it by [V_lo | V_hi] (value width 2*KEY_DIM).
//
// Work decomposition (ours, not the page's one-program-per-query-row): one
// workgroup per (batch-head, tile of 32*kWaves queries); each wave owns 32
// queries and walks all keys in tiles of 64, staged in LDS in the tensors' own
// layout and double-buffered (the next tile's loads are in flight while the
// current tile is computed). NCHW tiles with N a multiple of 8 go from global
// memory straight into LDS (buffer loads with an LDS destination, no registers
// on the way); the others pass through registers.
//
// Tail split: a grid rarely fills the chip's workgroup slots a whole number of
// times, and the last partial round would run on a few CUs while the rest idle.
// Those last query tiles are instead cut into key-range pieces, each an
// ordinary workgroup that stores its unnormalised O^T with its running max and
// sum; a small second kernel merges the pieces with the usual log-sum-exp
// weights and writes those tiles' outputs.
//
// Per wave and key tile, on the matrix cores (v_mfma_f32_32x32x16_bf16):
//   S^T[key][query] = K Q^T      A = K (LDS), B = Q (registers, loaded once)
//   O^T[dv][query] += V^T P^T    A = V^T (LDS), B = P (registers)
// With the transposed products each lane column is one query, so the running
// max and sum are per-lane scalars, and the S^T accumulator is already the
// B operand P of the second product: P never leaves registers.
//
// Operand reads. An MFMA operand needs 8 consecutive reduction-index values
// per lane. Where the LDS tile has the other index contiguous (K from NCHW
// channel rows, V from [n, D] rows), the operand comes from two
// ds_read_b64_tr_b16: inside each 16-lane group, lane i receives element i%4 of
// the 8 bytes addressed by lane 4r + i/4, for r = 0..3 -- a 4x16 transpose.
// The rows of S^T are also permuted (row 8h + 4g + e of each 16-row half holds
// key 8g + 4h + e): the accumulator rows a lane holds for one 16-key step are
// then 8 consecutive keys, so the V^T operand from NCHW channel rows is one
// 16-byte read.
//
// Softmax runs in base 2 with scale*log2(e) folded into one multiply-add; the
// running max is only moved when a tile's max exceeds it by more than 8 (so
// P <= 2^8), which skips most rescales of O. P is rounded to bf16 for the PV
// product and the row sum adds the same rounded values.
#include <math.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "psa_device.hpp"
#include "psa_launch.hpp"

namespace psa {
namespace {

constexpr int kBN = 64;   // keys per tile
constexpr int kWavesFwd = 4;   // waves per workgroup, 32 queries each
constexpr int kPad = 8;   // bf16 elements of padding per LDS row (spreads banks)

struct FwdArgs {
  const uint16_t* q;   // packed: [BH, n_q, KD]; NCHW: the qkv tensor
  const uint16_t* k;   // packed: [BH, n_k, KD]; NCHW: the qkv tensor
  const uint16_t* v;   // packed: [BH, n_k, DV]; NCHW: the qkv tensor
  uint16_t* o;         // packed: [BH, n_q, DV]; NCHW: out [BH*DV, N]
  uint16_t* vres;      // NCHW only: V residual [BH*DV, N], or null
  float* lse;          // [BH, n_q] or null
  int BH, n_q, n_k;
  int q_tiles;
  float c;             // scale * log2(e)
  int full;            // workgroups [0, full) each own a whole query tile
  int tail;            // query tiles split into key-range pieces (after them)
  int splits;          // pieces per split tile
  float* part;         // per piece: O^T [DV][BM] (unnormalised), m [BM], l [BM]
  int vres_wgs;        // > 0: workgroups after the attention ones copy the V residual
};

// Logical query tiles L = bh * q_tiles + qt in XCD-aware order. Workgroups are
// dispatched round-robin over the 8 XCDs (block i runs on XCD i % 8), so XCD x
// is given the contiguous run of tiles [x * per, (x + 1) * per): the query
// tiles of a batch-head share one L2 and its K/V stay resident there. When
// the tail is split, the split tiles are the last tail / 8 of every XCD's run
// and their pieces are dispatched on that same XCD. (Grids whose tile counts
// are not multiples of 8 use a plainer order.)
__device__ __forceinline__ bool xcd_order(const FwdArgs& a) {
  return (a.full + a.tail) % 8 == 0 && a.tail % 8 == 0;
}

// Tile of whole-tile workgroup i (i < full).
__device__ __forceinline__ int full_tile(const FwdArgs& a, int i) {
  if (xcd_order(a)) return (i % 8) * ((a.full + a.tail) / 8) + i / 8;
  const int per = a.full / 8;
  return (i < per * 8) ? (i % 8) * per + i / 8 : i;
}

// Tile of split tile s (0 <= s < tail); split tile s runs on XCD s % 8.
__device__ __forceinline__ int split_tile(const FwdArgs& a, int s) {
  if (xcd_order(a)) {
    const int per = (a.full + a.tail) / 8;
    return (s % 8) * per + (per - a.tail / 8) + s / 8;
  }
  return a.full + s;
}

// Value of x held by lane ^ 32 (g = lane / 32): one v_permlane32_swap, which
// leaves the partner's value in the first result on the upper half-wave and
// in the second on the lower.
__device__ __forceinline__ float lane_xor32(float x, int g) {
  const u32x2 sw = __builtin_bit_cast(u32x2, __builtin_amdgcn_permlane32_swap(
      __builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x), false, false));
  return __builtin_bit_cast(float, g ? sw[0] : sw[1]);
}

// Position of 16-byte chunk c of K channel row `row` in a directly staged
// NCHW key tile (64 keys = 8 chunks per row). The transposed K reads of one
// 32-lane half take chunks 4kb..4kb+3 of four consecutive rows; flipping
// chunk bit 2 on rows 2 and 3 of every four puts those 256 bytes on all 64
// banks (unswizzled, rows r and r + 2 share their banks).
__device__ __forceinline__ int k_chunk_pos(int row, int c) { return c ^ (((row >> 1) & 1) << 2); }

// Whether a kernel instance stages its tiles straight into LDS: NCHW tiles
// with N a multiple of 8, packed tiles with head dim 32..128 (kVecN then means
// the rows fit the buffer offsets).
template <int KD, bool kNCHW, bool kVecN>
constexpr bool direct_staging() {
  return kVecN && (kNCHW || KD >= 32);
}

template <int KD, int DV, bool kNCHW, int kWaves, bool kDirect>
struct FwdCfg {
  static constexpr int NT = kWaves * 64;
  static constexpr int BM = 32 * kWaves;                   // queries per workgroup
  static constexpr int DVP = DV < 32 ? 32 : DV;            // O^T rows (one MFMA block minimum)
  // NCHW: K as [KD][keys], V as [DV][keys]. packed: K as [keys][KD], V as [keys][DVP].
  // Direct (global -> LDS) staging writes whole 1 KB runs, so its rows are unpadded.
  static constexpr int PAD = kDirect ? 0 : kPad;
  static constexpr int KROW = kNCHW ? kBN + PAD : KD + PAD;
  static constexpr int VROW = kNCHW ? kBN + PAD : DVP + PAD;
  static constexpr int K_ROWS = kNCHW ? KD : kBN;
  static constexpr int V_ROWS = kNCHW ? DV : kBN;
  static constexpr int K_ELEMS = K_ROWS * KROW;
  static constexpr int V_ELEMS = V_ROWS * VROW;
  static constexpr int BUF = K_ELEMS + V_ELEMS;
  static constexpr int K_CPR = (kNCHW ? kBN : KD) / 8;     // 16-byte chunks per LDS row
  static constexpr int V_CPR = (kNCHW ? kBN : DV) / 8;
  static constexpr int K_CH = K_ROWS * K_CPR;
  static constexpr int V_CH = V_ROWS * V_CPR;
  static constexpr int PER = (K_CH + V_CH + NT - 1) / NT;  // chunks per thread per tile
  static constexpr int PART = (DV + 2) * BM;               // floats per split piece
};

// Tail split limits: at most kMaxSplits pieces per query tile, each of at
// least kSplitMinTiles key tiles (shorter pieces do not repay their extra
// partial-result traffic and the merge).
constexpr int kMaxSplits = 6;
constexpr int kSplitMinTiles = 16;

// Direct global -> LDS staging of one NCHW key tile (N a multiple of 8): each
// wave instruction (buffer_load_dwordx4 ... lds) fills 64 consecutive 16-byte LDS
// chunks, lane i the i-th; lanes pick which global chunk to fetch, which is
// how the V swizzle is applied. No registers and no LDS write instructions;
// the wave waits with vmcnt before the barrier that publishes the tile.
template <int KD, int DV, int kWaves>
struct FwdStageDirect {
  static constexpr int K_BLOCKS = KD * (kBN / 8) / 64;     // 1 KB blocks of K
  static constexpr int V_BLOCKS = DV * (kBN / 8) / 64;     // 1 KB blocks of V
  static constexpr int BLOCKS = K_BLOCKS + V_BLOCKS;
  static constexpr int PER = (BLOCKS + kWaves - 1) / kWaves;   // blocks per wave
  static_assert(KD * (kBN / 8) % 64 == 0 && DV * (kBN / 8) % 64 == 0, "whole 1 KB blocks");

  // Block b covers 8 channel rows starting at chan0(b) of the batch-head's
  // [4*KD][N] slab; lane i fills LDS chunk i of it: row i/8 of the block, and
  // the 8 keys the swizzle puts at position i%8 (k_chunk_pos for K rows,
  // tile_chunk_pos for V rows; both are their own inverses).
  __device__ static int chan0(int b) { return b < K_BLOCKS ? KD + 8 * b : 2 * KD + 8 * (b - K_BLOCKS); }
  __device__ static int chunk(int b, int lane) {
    const int r = lane >> 3;
    return b < K_BLOCKS ? k_chunk_pos(8 * b + r, lane & 7) : tile_chunk_pos(8 * (b - K_BLOCKS) + r, lane & 7);
  }

  uint32_t voff[PER];   // byte offset of this lane's 16 bytes from the block's (row, key) origin

  __device__ __forceinline__ void init(int N, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int b = wave + i * kWaves;
      voff[i] = b < BLOCKS ? static_cast<uint32_t>((lane >> 3) * N + chunk(b, lane) * 8) * 2u : 0u;
    }
  }

  // `wave` must be wave-uniform (an SGPR value). Tiles are fetched with buffer
  // loads over the batch-head's [4*KD][N] slab (under 2 GB: the launcher
  // checks): for a whole tile the lane's offset voff[i] is the same for every
  // tile and the block's (channel, key) origin is a scalar offset, so issuing
  // costs no vector instructions. The last, partial tile clamps its keys to
  // real data (their scores are masked later).
  __device__ __forceinline__ void issue(const FwdArgs& a, int bh, int kt, int wave, int lane,
                                        uint16_t* buf) const {
    const int N = a.n_k;
    const int m0 = kt * kBN;
    const bool last = m0 + kBN > N;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(a.k + static_cast<int64_t>(bh) * 4 * KD * N), 0, 4 * KD * N * 2,
        kBufferWord3);
    if (!last) {   // whole tile: per-lane offsets as set up by init(), tile origin scalar
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int b = wave + i * kWaves;
        if (BLOCKS % kWaves != 0 && b >= BLOCKS) break;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rsrc, (__attribute__((address_space(3))) void*)(buf + b * 512), 16, voff[i],
            (chan0(b) * N + m0) * 2, 0, 0);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int b = wave + i * kWaves;
      if (BLOCKS % kWaves != 0 && b >= BLOCKS) break;
      int m = m0 + chunk(b, lane) * 8;
      m = m < N ? m : N - 8;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsrc, (__attribute__((address_space(3))) void*)(buf + b * 512), 16,
          static_cast<uint32_t>((lane >> 3) * N + m) * 2u, chan0(b) * N * 2, 0, 0);
    }
  }
};

// Direct global -> LDS staging of one packed key tile ([BH, n, D] K and V,
// D >= 32): 64 rows of D elements each, unpadded, chunks placed by
// packed_chunk_pos. Wave instruction b fills one 1 KB block (512 / D rows);
// lane i fetches the global chunk the swizzle puts at LDS chunk i. Buffer
// loads over one batch-head's [n_k][D] rows (under 2 GB: the launcher checks):
// for a whole tile the lane's offset is the same for every tile and the
// tile's first row is a scalar offset. The last, partial tile repeats row
// n_k - 1 (its scores are masked).
template <int KD, int DV, int kWaves>
struct FwdStagePacked {
  static_assert(KD == DV, "packed direct staging serves fa2_fwd (value width = head dim)");
  static constexpr int CPR = KD / 8;                       // chunks per row
  static constexpr int RPB = 64 / CPR;                     // rows per 1 KB block
  static constexpr int K_BLOCKS = kBN / RPB;
  static constexpr int BLOCKS = 2 * K_BLOCKS;              // K blocks, then V blocks
  static constexpr int PER = (BLOCKS + kWaves - 1) / kWaves;

  __device__ static int row_of(int b, int lane) { return (b % K_BLOCKS) * RPB + lane / CPR; }
  __device__ static int chunk_of(int b, int lane) {
    return packed_chunk_pos<KD>(row_of(b, lane), lane % CPR);   // the swizzle is an involution
  }

  uint32_t voff[PER];   // byte offset of this lane's 16 bytes from the tile's first row

  __device__ __forceinline__ void init(int /*N*/, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int b = wave + i * kWaves;
      voff[i] = b < BLOCKS ? static_cast<uint32_t>(row_of(b, lane) * KD + chunk_of(b, lane) * 8) * 2u : 0u;
    }
  }

  __device__ __forceinline__ void issue(const FwdArgs& a, int bh, int kt, int wave, int lane,
                                        uint16_t* buf) const {
    const int n = a.n_k;
    const int m0 = kt * kBN;
    const bool last = m0 + kBN > n;
    const int64_t base = static_cast<int64_t>(bh) * n * KD;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(a.k + base), 0, n * KD * 2, kBufferWord3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(a.v + base), 0, n * KD * 2, kBufferWord3);
    if (!last) {   // whole tile: per-lane offsets as set up by init(), tile origin scalar
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int b = wave + i * kWaves;
        if (BLOCKS % kWaves != 0 && b >= BLOCKS) break;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            b < K_BLOCKS ? rk : rv, (__attribute__((address_space(3))) void*)(buf + b * 512), 16, voff[i],
            m0 * KD * 2, 0, 0);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int b = wave + i * kWaves;
      if (BLOCKS % kWaves != 0 && b >= BLOCKS) break;
      const int r = row_of(b, lane);
      const int m = m0 + r < n ? r : n - 1 - m0;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          b < K_BLOCKS ? rk : rv, (__attribute__((address_space(3))) void*)(buf + b * 512), 16,
          static_cast<uint32_t>(m * KD + chunk_of(b, lane) * 8) * 2u, m0 * KD * 2, 0, 0);
    }
  }
};

// Global -> registers -> LDS staging of one key tile (K and V), 16-byte chunks.
// Keys past n_k are clamped to real rows (finite data): their scores are
// masked to -inf, so they contribute nothing. The unaligned NCHW variant
// (N not a multiple of 8) gathers element by element and zero-fills instead.
template <int KD, int DV, bool kNCHW, bool kVecN, int kWaves>
struct FwdStage {
  using C = FwdCfg<KD, DV, kNCHW, kWaves, false>;
  u32x4 r[C::PER];

  __device__ __forceinline__ void load(const FwdArgs& a, int bh, int kt, int tid) {
    const int m0 = kt * kBN;
#pragma unroll
    for (int i = 0; i < C::PER; ++i) {
      const int c = tid + i * C::NT;
      if (c >= C::K_CH + C::V_CH) continue;
      const bool is_k = c < C::K_CH;
      const int cc = is_k ? c : c - C::K_CH;
      const int row = cc / (is_k ? C::K_CPR : C::V_CPR);
      const int col = cc - row * (is_k ? C::K_CPR : C::V_CPR);
      if constexpr (kNCHW) {
        const int N = a.n_k;
        const int m = m0 + col * 8;
        const int64_t ch = static_cast<int64_t>(bh) * 4 * KD + (is_k ? KD : 2 * KD) + row;
        if constexpr (kVecN)
          r[i] = load16(a.k + ch * N + (m < N ? m : N - 8));
        else
          r[i] = gather8(a.k + ch * N + m, 1, m, N);
      } else {
        int m = m0 + row;
        m = m < a.n_k ? m : a.n_k - 1;
        const int64_t rowi = static_cast<int64_t>(bh) * a.n_k + m;
        r[i] = is_k ? load16(a.k + rowi * KD + col * 8) : load16(a.v + rowi * DV + col * 8);
      }
    }
  }

  __device__ __forceinline__ void store(uint16_t* buf, int tid) const {
#pragma unroll
    for (int i = 0; i < C::PER; ++i) {
      const int c = tid + i * C::NT;
      if (c >= C::K_CH + C::V_CH) continue;
      const bool is_k = c < C::K_CH;
      const int cc = is_k ? c : c - C::K_CH;
      const int row = cc / (is_k ? C::K_CPR : C::V_CPR);
      const int col = cc - row * (is_k ? C::K_CPR : C::V_CPR);
      uint16_t* dst = is_k ? buf + row * C::KROW + col * 8 : buf + C::K_ELEMS + row * C::VROW + col * 8;
      *reinterpret_cast<u32x4*>(dst) = r[i];
    }
  }
};

// ---- pieces of the forward kernel (NCHW and packed)

// V residual workgroups (NCHW, N a multiple of 8): queued after every
// attention workgroup, they run on the slots the grid's last partial round
// leaves free. A batch-head's V channels are DV*N contiguous elements on both
// sides, so the residual is a plain copy of BH such blocks. Workgroup w
// (counted from the first residual workgroup) copies every vres_wgs-th chunk.
template <int KD, int DV, int NT>
__device__ __forceinline__ void vres_copy_wg(const FwdArgs& a, int N, int w, int tid) {
  const int64_t per_bh = static_cast<int64_t>(DV) * N / 8;   // 16-byte chunks
  const int64_t total = per_bh * a.BH;
  const int64_t stride = static_cast<int64_t>(a.vres_wgs) * NT;
  constexpr int BATCH = 8;
  for (int64_t c0 = static_cast<int64_t>(w) * NT + tid; c0 < total; c0 += stride * BATCH) {
    u32x4 r[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int64_t c = min(c0 + u * stride, total - 1);
      const int64_t bh_c = c / per_bh;
      r[u] = ldg_nt(reinterpret_cast<const u32x4*>(a.v + (bh_c * 4 * KD + 2 * KD) * N + (c - bh_c * per_bh) * 8));
    }
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int64_t c = c0 + u * stride;
      const int64_t bh_c = c / per_bh;
      if (c < total) stg_nt(reinterpret_cast<u32x4*>(a.vres + bh_c * DV * N + (c - bh_c * per_bh) * 8), r[u]);
    }
  }
}

// Work unit of attention workgroup i: a whole query tile (split = -1), or key
// tiles [kt0, kt1) (piece `piece`) of split tile `split`. L is the logical
// query tile.
__device__ __forceinline__ void work_unit(const FwdArgs& a, int i, int n_tiles, int& L, int& split, int& piece,
                                          int& kt0, int& kt1) {
  split = -1;
  piece = 0;
  kt0 = 0;
  kt1 = n_tiles;
  if (i < a.full) {
    L = full_tile(a, i);
    return;
  }
  const int j = i - a.full;   // pieces of one split tile stay on one XCD
  if (xcd_order(a)) {
    const int local = j / 8;
    split = (local / a.splits) * 8 + j % 8;
    piece = local % a.splits;
  } else {
    split = j / a.splits;
    piece = j % a.splits;
  }
  L = split_tile(a, split);
  kt0 = piece * n_tiles / a.splits;
  kt1 = (piece + 1) * n_tiles / a.splits;
}

// V residual of one query tile (NCHW, N a multiple of 8): this tile's pixel
// columns of the V channels. The loads of a batch are unconditional (chunks
// past the map's last pixel re-read its last chunk; only the stores are
// guarded), so they are all in flight together.
template <int KD, int DV, int NT, int BM>
__device__ __forceinline__ void vres_copy_tile(const FwdArgs& a, int bh, int qt, int N, int tid) {
  const int n0 = qt * BM;
  constexpr int CPR = BM / 8;   // 8-pixel chunks per channel row
  constexpr int TOTAL = DV * CPR;
  static_assert(TOTAL % NT == 0, "V residual chunks per thread");
  constexpr int PER = TOTAL / NT;
  constexpr int BATCH = PER < 8 ? PER : 8;
#pragma unroll
  for (int u0 = 0; u0 < PER; u0 += BATCH) {
    u32x4 r[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int c = (u0 + u) * NT + tid, dv = c / CPR, n = n0 + (c % CPR) * 8;
      r[u] = load16(a.v + (static_cast<int64_t>(bh) * 4 * KD + 2 * KD + dv) * N + min(n, N - 8));
    }
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int c = (u0 + u) * NT + tid, dv = c / CPR, n = n0 + (c % CPR) * 8;
      if (n < N) stg_nt(reinterpret_cast<u32x4*>(a.vres + (static_cast<int64_t>(bh) * DV + dv) * N + n), r[u]);
    }
  }
}

// End of a work unit. A whole query tile: O = O^T / l in bf16, LSE =
// (m + log2 l) ln 2. A piece of a split tile: its unnormalised O^T, running
// max and sum, for the merge kernel. ql = this lane's query within the tile.
template <int DV, int NDB, int BM, int PART, bool kNCHW>
__device__ __forceinline__ void store_result(const FwdArgs& a, const f32x16 (&oacc)[NDB], float m_run, float l_tot,
                                             int bh, int q_row, bool q_ok, int split, int piece, int ql, int g) {
  const int N = a.n_k;
  if (split < 0) {
    const float inv = 1.0f / l_tot;
    if (!q_ok) return;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int dv0 = db * 32 + 8 * r4 + 4 * g;
        if (dv0 >= DV) continue;
        uint16_t h[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = float_to_bf16_bits(oacc[db][4 * r4 + e] * inv);
        if constexpr (kNCHW) {
          uint16_t* dst = a.o + (static_cast<int64_t>(bh) * DV + dv0) * N + q_row;
#pragma unroll
          for (int e = 0; e < 4; ++e) dst[static_cast<int64_t>(e) * N] = h[e];
        } else {
          uint16_t* dst = a.o + (static_cast<int64_t>(bh) * a.n_q + q_row) * DV + dv0;
          *reinterpret_cast<u32x2*>(dst) = u32x2{h[0] | (uint32_t(h[1]) << 16), h[2] | (uint32_t(h[3]) << 16)};
        }
      }
    if (a.lse != nullptr && g == 0)
      a.lse[static_cast<int64_t>(bh) * a.n_q + q_row] = (m_run + log2f(l_tot)) * kLn2;
    return;
  }
  float* pp = a.part + (static_cast<int64_t>(split) * a.splits + piece) * PART;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int dv0 = db * 32 + 8 * r4 + 4 * g;
      if (dv0 >= DV) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) pp[(dv0 + e) * BM + ql] = oacc[db][4 * r4 + e];
    }
  if (g == 0) {
    pp[DV * BM + ql] = m_run;
    pp[DV * BM + BM + ql] = l_tot;
  }
}

// kOcc: waves per SIMD the register allocation must allow.
template <int KD, int DV, bool kNCHW, bool kVecN, int kWaves, int kOcc>
__global__ __launch_bounds__(kWaves * 64, kOcc) void attn_fwd_bf16(FwdArgs a) {
  constexpr bool kDirect = direct_staging<KD, kNCHW, kVecN>();
  using C = FwdCfg<KD, DV, kNCHW, kWaves, kDirect>;
  constexpr int NT = C::NT;
  constexpr int BM = C::BM;
  constexpr int NKB = kBN / 32;        // 32-key blocks per tile
  constexpr int NKS = kBN / 16;        // 16-key MFMA steps per tile
  constexpr int NDS = KD / 16;         // 16-wide d steps of K Q^T
  constexpr int NDB = C::DVP / 32;     // 32-row blocks of O^T
  // Two tile buffers as two objects: the compiler can then tell that the
  // direct global->LDS loads into one do not alias the LDS reads of the other,
  // and does not make those reads wait for the loads.
  __shared__ __attribute__((aligned(16))) uint16_t smem0[C::BUF];
  __shared__ __attribute__((aligned(16))) uint16_t smem1[C::BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int g = lane >> 5;           // lane group of the MFMA layouts
  const int i16 = lane & 15;         // lane inside its 16-lane group
  const int t16 = (lane >> 4) & 1;   // which 16-row half of an operand block
  const int N = a.n_k;   // NCHW: n_q == n_k == H*W
  const int n_tiles = (a.n_k + kBN - 1) / kBN;

  // V residual workgroups (NCHW, N a multiple of 8): queued after every
  // attention workgroup, they run on the slots the grid's last partial round
  // leaves free. A batch-head's V channels are DV*N contiguous elements on
  // both sides, so the residual is a plain copy of BH such blocks.
  if constexpr (kNCHW && kVecN) {
    const int n_attn = a.full + a.tail * a.splits;
    if (a.vres_wgs > 0 && static_cast<int>(blockIdx.x) >= n_attn) {
      vres_copy_wg<KD, DV, NT>(a, N, static_cast<int>(blockIdx.x) - n_attn, tid);
      return;
    }
  }

  int L, split, piece, kt0, kt1;
  work_unit(a, blockIdx.x, n_tiles, L, split, piece, kt0, kt1);
  const int bh = L / a.q_tiles;
  const int qt = L - bh * a.q_tiles;
  const int q_row = qt * BM + wave * 32 + l32;
  const bool q_ok = q_row < a.n_q;
  const bool wave_live = qt * BM + wave * 32 < a.n_q;   // uniform across the wave

  // Packed V with DV = 16: columns 16..31 of every V row stay zero in both buffers.
  if constexpr (!kNCHW && !kDirect && C::DVP > DV) {
    for (int e = tid; e < kBN * (C::DVP - DV); e += NT) {
      const int row = e / (C::DVP - DV), col = DV + e % (C::DVP - DV);
      smem0[C::K_ELEMS + row * C::VROW + col] = 0;
      smem1[C::K_ELEMS + row * C::VROW + col] = 0;
    }
  }

  // The first key tile's direct loads go out first, so that their round trip
  // overlaps the V residual copy and the Q loads below.
  FwdStage<KD, DV, kNCHW, kVecN, kWaves> stage;
  using DirectStage = typename std::conditional<kNCHW, FwdStageDirect<KD, DV, kWaves>,
                                                 FwdStagePacked<KD, (kNCHW ? KD : DV), kWaves>>::type;
  DirectStage dstage;
  if constexpr (kDirect) {
    dstage.init(N, wave, lane);
    dstage.issue(a, bh, kt0, wave, lane, smem0);
  }

  // V residual: copy this tile's pixel columns of the V channels (NCHW only;
  // the first piece of a split tile does it).
  if constexpr (kNCHW) {
    if (a.vres != nullptr && piece == 0 && a.vres_wgs == 0) {
      if constexpr (kVecN) {
        vres_copy_tile<KD, DV, NT, BM>(a, bh, qt, N, tid);
      } else {
        const int n0 = qt * BM;
        constexpr int CPR = BM / 8;   // 8-pixel chunks per channel row
        constexpr int TOTAL = DV * CPR;
        for (int c = tid; c < TOTAL; c += NT) {
          const int dv = c / CPR, n = n0 + (c % CPR) * 8;
          const uint16_t* src = a.v + (static_cast<int64_t>(bh) * 4 * KD + 2 * KD + dv) * N + n;
          uint16_t* dst = a.vres + (static_cast<int64_t>(bh) * DV + dv) * N + n;
          for (int e = 0; e < 8; ++e)
            if (n + e < N) dst[e] = src[e];
        }
      }
    }
  }

  // This lane's Q operands: Q[q_row][16*ds + 8*g + j], j = 0..7. Rows past
  // n_q load row n_q - 1 (every load unconditional, all in flight together)
  // and are zeroed afterwards.
  bf16x8 qop[NDS];
  {
    const int qr = min(q_row, a.n_q - 1);
    u32x4 raw[NDS];
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      if constexpr (kNCHW)
        raw[ds] = gather8(a.q + (static_cast<int64_t>(bh) * 4 * KD + ds * 16 + g * 8) * N + qr, N, 0, 8);
      else
        raw[ds] = load16(a.q + (static_cast<int64_t>(bh) * a.n_q + qr) * KD + ds * 16 + g * 8);
    }
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) qop[ds] = as_bf16x8(q_ok ? raw[ds] : zero4());
  }

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;
  float m_run = -INFINITY;   // running max of scale*log2(e)*S
  float m_thr = -INFINITY;   // (m_run + 8) / (scale*log2(e)): the rescale threshold on raw scores
  const float inv_c = 1.0f / a.c;
  float l_run = 0.0f;        // this lane's part of the running sum (its lane group's keys)
  // At key_dim 32 the VALU work per score outweighs the MFMA work, so the row
  // sums go to the matrix cores instead: one 16x16x32 MFMA per 16-key step
  // multiplies a selector (row 0 picks the B rows of queries 0..15, row 1 those
  // of queries 16..31) by the step's P operand as laid out for the PV product.
  // Lane n < 16 then holds the running sum of query n in element 0 and of
  // query 16 + n in element 1; every other accumulator element stays zero.
  constexpr bool kSumMfma = KD == 32;
  f32x4 lacc = {0.0f, 0.0f, 0.0f, 0.0f};
  bf16x8 lsel;
  {
    const __bf16 on = static_cast<__bf16>((lane & 15) == ((lane >> 4) & 1) ? 1.0f : 0.0f);
#pragma unroll
    for (int j = 0; j < 8; ++j) lsel[j] = on;
  }

  if constexpr (kDirect) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's part of tile kt0 landed
  } else {
    stage.load(a, bh, kt0, tid);
    stage.store(smem0, tid);
  }
  __syncthreads();

  // One key tile: computes from ks while the next tile is loaded into nbuf.
  auto tile = [&](int kt, const uint16_t* __restrict__ ks, uint16_t* __restrict__ nbuf)
                  __attribute__((always_inline)) {
    const uint16_t* vs = ks + C::K_ELEMS;
    const bool more = kt + 1 < kt1;
    if constexpr (kDirect) {
      if (more) dstage.issue(a, bh, kt + 1, wave, lane, nbuf);
    } else {
      if (more) stage.load(a, bh, kt + 1, tid);
    }

    // A wave whose 32 queries all lie past n_q (the last query tile of a
    // batch-head when n_q is not a multiple of the tile) only helps stage
    // the tiles and meets the barriers.
    if (wave_live) {
      // S^T = K Q^T for the tile's keys (rows permuted by key_of_row).
      f32x16 sacc[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.0f;
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) {
          bf16x8 kop;
          if constexpr (kNCHW && kDirect) {
            // Rows row and row + 4 of the two reads share the swizzle.
            const int row = ds * 16 + 8 * g + (i16 >> 2);
            const int col = kb * 32 + 16 * t16 + tr_key_col(i16 & 3);
            kop = lds_read_tr8(ks + row * C::KROW + k_chunk_pos(row, col >> 3) * 8 + (col & 7), C::KROW);
          } else if constexpr (kNCHW)
            kop = lds_read_tr8(ks + (ds * 16 + 8 * g + (i16 >> 2)) * C::KROW + kb * 32 + 16 * t16 +
                                   tr_key_col(i16 & 3), C::KROW);
          else if constexpr (kDirect) {
            const int row = kb * 32 + key_of_row(l32);
            kop = *reinterpret_cast<const bf16x8*>(ks + row * C::KROW + packed_chunk_pos<KD>(row, ds * 2 + g) * 8);
          } else
            kop = *reinterpret_cast<const bf16x8*>(ks + (kb * 32 + key_of_row(l32)) * C::KROW + ds * 16 + g * 8);
          sacc[kb] = mfma32x32x16(kop, qop[ds], sacc[kb]);
        }
      }
      // Keys past n_k (last tile only) get -inf. Element r of block kb holds
      // key 32*kb + 16*(r/8) + 8*g + r%8 of the tile.
      if ((kt + 1) * kBN > a.n_k) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kt * kBN + kb * 32 + 16 * (r >> 3) + 8 * g + (r & 7);
            if (key >= a.n_k) sacc[kb][r] = -INFINITY;
          }
      }

      // Online softmax: running max, rescale, P = 2^(c*S - m).
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
      // The running max only moves when some lane's tile max exceeds it by more
      // than 8 (log2 units): until then P <= 2^8, harmless in fp32 and bf16. The
      // test is on the raw scores, against the threshold kept since the last move.
      // A query's keys are split between lanes l and l ^ 32, which hold the same
      // threshold, so testing each lane's own half decides exactly as testing the
      // whole row would; the row max itself is only needed when the max moves.
      if (__any(mx > m_thr)) {
        mx = fmaxf(mx, lane_xor32(mx, g));
        const float m_new = fmaxf(m_run, mx * a.c);
        const float alpha = fast_exp2(m_run - m_new);
        m_run = m_new;
        m_thr = (m_run + 8.0f) * inv_c;
        if constexpr (kSumMfma) {
          lacc[0] *= __shfl(alpha, lane & 15);
          lacc[1] *= __shfl(alpha, (lane & 15) + 16);
        } else {
          l_run *= alpha;
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      }

      bf16x8 pop[NKS];
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          pop[s][j] = static_cast<__bf16>(fast_exp2(fmaf(sacc[s >> 1][8 * (s & 1) + j], a.c, -m_run)));
        if constexpr (kSumMfma) {
          lacc = mfma16x16x32(lsel, pop[s], lacc);
        } else {
#pragma unroll
          for (int j = 0; j < 8; j += 2) {
            const bf16x2 pp = {pop[s][j], pop[s][j + 1]};
            l_run = __builtin_amdgcn_fdot2_f32_bf16(pp, bf16x2{1.0f, 1.0f}, l_run, false);
          }
        }
      }

      // O^T += V^T P^T: step s covers keys 16s + 8g + j of the tile in this lane's P.
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
          bf16x8 vop;
          if constexpr (kDirect && kNCHW)
            vop = *reinterpret_cast<const bf16x8*>(vs + (db * 32 + l32) * C::VROW +
                                                   tile_chunk_pos(db * 32 + l32, 2 * s + g) * 8);
          else if constexpr (kDirect) {
            // Two transposed reads, rows r and r + 4, each at its own swizzled chunk.
            const int r = s * 16 + 8 * g + (i16 >> 2);
            const int col = db * 32 + 16 * t16 + 4 * (i16 & 3);
            vop = lds_read_tr8_2(vs + r * C::VROW + packed_chunk_pos<DV>(r, col >> 3) * 8 + (col & 7),
                                 vs + (r + 4) * C::VROW + packed_chunk_pos<DV>(r + 4, col >> 3) * 8 + (col & 7));
          } else if constexpr (kNCHW)
            vop = *reinterpret_cast<const bf16x8*>(vs + (db * 32 + l32) * C::VROW + s * 16 + g * 8);
          else
            vop = lds_read_tr8(vs + (s * 16 + 8 * g + (i16 >> 2)) * C::VROW + db * 32 + 16 * t16 + 4 * (i16 & 3),
                               C::VROW);
          oacc[db] = mfma32x32x16(vop, pop[s], oacc[db]);
        }
    }

    if constexpr (kDirect) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's part of tile kt+1 landed
    } else {
      if (more) stage.store(nbuf, tid);
    }
    __syncthreads();
  };

  // Tile kt0 + 2i lives in smem0, kt0 + 2i + 1 in smem1. Up to key_dim 64 the
  // loop takes two tiles per trip, so that each tile's LDS buffers are fixed
  // objects: every operand address is then a loop-invariant per-lane offset
  // plus an immediate (key_dim 128 has no registers to spare for the second
  // set of addresses).
  if constexpr (KD <= 64) {
    int kt = kt0;
    for (; kt + 1 < kt1; kt += 2) {
      tile(kt, smem0, smem1);
      tile(kt + 1, smem1, smem0);
    }
    if (kt < kt1) tile(kt, smem0, smem1);
  } else {
    for (int kt = kt0; kt < kt1; ++kt) {
      const bool odd = (kt - kt0) & 1;
      tile(kt, odd ? smem1 : smem0, odd ? smem0 : smem1);
    }
  }

  float l_tot;
  if constexpr (kSumMfma) {
    const float s0 = __shfl(lacc[0], l32 & 15), s1 = __shfl(lacc[1], l32 & 15);
    l_tot = l32 < 16 ? s0 : s1;
  } else {
    l_tot = l_run + lane_xor32(l_run, g);
  }
  store_result<DV, NDB, BM, C::PART, kNCHW>(a, oacc, m_run, l_tot, bh, q_row, q_ok, split, piece, wave * 32 + l32, g);
}

// Merge of split tiles. One workgroup per (split tile, 8 rows of O^T); each
// thread owns 4 consecutive queries of one row. Per query, with M the largest
// piece max m_c: w_c = 2^(m_c - M) / sum_c 2^(m_c - M) l_c, O = sum_c w_c O_c,
// LSE = (M + log2 sum_c 2^(m_c - M) l_c) ln 2. Every load of a thread is
// independent of the others, so the merge costs one or two memory round trips.
constexpr int kMergeThreads = 256;

template <int DV, bool kNCHW, int BM, int PART>
__global__ __launch_bounds__(kMergeThreads) void attn_fwd_merge(FwdArgs a) {
  constexpr int QV = BM / 4;                   // 4-query groups per row
  constexpr int ROWS = kMergeThreads / QV;     // O^T rows per workgroup
  constexpr int CHUNKS = DV / ROWS;
  static_assert(kMergeThreads % QV == 0 && DV % ROWS == 0, "merge tiling");
  const int split = blockIdx.x / CHUNKS;
  const int dv = (blockIdx.x - split * CHUNKS) * ROWS + threadIdx.x / QV;
  const int q4 = (threadIdx.x % QV) * 4;
  const int L = split_tile(a, split);
  const int bh = L / a.q_tiles;
  const int qt = L - bh * a.q_tiles;
  const int S = a.splits;
  const float* part0 = a.part + static_cast<int64_t>(split) * S * PART;

  f32x4 m[kMaxSplits], l[kMaxSplits], o[kMaxSplits];
#pragma unroll
  for (int c = 0; c < kMaxSplits; ++c) {
    if (c < S) {
      const float* pc = part0 + c * PART;
      m[c] = *reinterpret_cast<const f32x4*>(pc + DV * BM + q4);
      l[c] = *reinterpret_cast<const f32x4*>(pc + DV * BM + BM + q4);
      o[c] = *reinterpret_cast<const f32x4*>(pc + dv * BM + q4);
    } else {
      m[c] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      l[c] = o[c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float M = m[0][e];
#pragma unroll
    for (int c = 1; c < kMaxSplits; ++c) M = fmaxf(M, m[c][e]);
    float sum = 0.0f, acc = 0.0f;
#pragma unroll
    for (int c = 0; c < kMaxSplits; ++c) {
      const float wc = fast_exp2(m[c][e] - M);   // 0 for pieces past S
      sum = fmaf(wc, l[c][e], sum);
      acc = fmaf(wc, o[c][e], acc);
    }
    const int row = qt * BM + q4 + e;
    if (row >= a.n_q) continue;
    const uint16_t h = float_to_bf16_bits(acc / sum);
    if constexpr (kNCHW)
      a.o[(static_cast<int64_t>(bh) * DV + dv) * a.n_k + row] = h;
    else
      a.o[(static_cast<int64_t>(bh) * a.n_q + row) * DV + dv] = h;
    if (dv == 0 && a.lse != nullptr)
      a.lse[static_cast<int64_t>(bh) * a.n_q + row] = (M + log2f(sum)) * kLn2;
  }
}

// ------------------------------------------------------------------ float32

struct FwdArgsF32 {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* vres;
  float* lse;
  int BH, n_q, n_k;
  float scale;
  int bh0;   // first batch-head of this launch
};

constexpr int kF32Threads = 128;
constexpr int kF32Keys = 32;                          // keys per LDS tile
constexpr int kF32Lanes = 4;                          // lanes per query row
constexpr int kF32Rows = kF32Threads / kF32Lanes;     // query rows per workgroup
constexpr int kF32Sub = kF32Keys / kF32Lanes;         // keys per lane and tile

// Four lanes per query row, keys staged through LDS in tiles of 32, float32
// throughout with expf. Lane l of a row takes keys l, l+4, ... of every tile
// and keeps its own online softmax (maximum, row sum, accumulator); its 8 keys
// of a tile are scored side by side and the maximum moves once per tile. The
// four partial softmaxes of a row are combined at the end (lane exchanges
// within the group of four), and each lane stores a quarter of the columns.
// The fused (NCHW) variant computes the softmax once and multiplies P by both
// V halves, [V_lo | V_hi] (value width 2*KD), as the bf16 kernel does, up to
// key_dim 64; at key_dim 128 (a 256-wide accumulator per lane would not fit
// the registers) workgroups take one V half each and the softmax is computed
// once per half. Workgroups enumerate (bh, V part, query block).
template <int KD, bool kNCHW>
constexpr int f32_parts() { return kNCHW && KD > 64 ? 2 : 1; }   // workgroups per (bh, query block)

template <int KD, bool kNCHW>
__global__ __launch_bounds__(kF32Threads) void attn_fwd_f32(FwdArgsF32 a) {
  constexpr int kParts = f32_parts<KD, kNCHW>();
  constexpr int VW = kNCHW && kParts == 1 ? 2 * KD : KD;   // value columns per workgroup
  __shared__ float ks[kF32Keys][KD];
  __shared__ float vs[kF32Keys][VW];
  const int q_blocks = (a.n_q + kF32Rows - 1) / kF32Rows;
  const int qb = blockIdx.x % q_blocks;
  const int bh = a.bh0 + static_cast<int>((blockIdx.x / q_blocks) / kParts);
  const int j = (blockIdx.x / q_blocks) % kParts;
  const int lane = threadIdx.x % kF32Lanes;
  const int row = qb * kF32Rows + threadIdx.x / kF32Lanes;
  const bool ok = row < a.n_q;
  const int N = a.n_k;
  // Element (row n, column d) of Q, K and this workgroup's V columns, in either layout.
  auto qi = [&](int n, int d) -> int64_t {
    return kNCHW ? (static_cast<int64_t>(bh) * 4 * KD + d) * N + n
                 : (static_cast<int64_t>(bh) * a.n_q + n) * KD + d;
  };
  auto ki = [&](int n, int d) -> int64_t {
    return kNCHW ? (static_cast<int64_t>(bh) * 4 * KD + KD + d) * N + n
                 : (static_cast<int64_t>(bh) * a.n_k + n) * KD + d;
  };
  auto vi = [&](int n, int d) -> int64_t {
    return kNCHW ? (static_cast<int64_t>(bh) * 4 * KD + 2 * KD + j * KD + d) * N + n
                 : (static_cast<int64_t>(bh) * a.n_k + n) * KD + d;
  };
  float q[KD], o[VW];
#pragma unroll
  for (int d = 0; d < KD; ++d) q[d] = ok ? a.q[qi(row, d)] : 0.0f;
#pragma unroll
  for (int d = 0; d < VW; ++d) o[d] = 0.0f;
  float m = -INFINITY, l = 0.0f;
  for (int m0 = 0; m0 < a.n_k; m0 += kF32Keys) {
    __syncthreads();
    for (int e = threadIdx.x; e < kF32Keys * KD; e += kF32Threads) {
      const int r = kNCHW ? e % kF32Keys : e / KD;
      const int d = kNCHW ? e / kF32Keys : e % KD;
      ks[r][d] = m0 + r < a.n_k ? a.k[ki(m0 + r, d)] : 0.0f;
    }
    for (int e = threadIdx.x; e < kF32Keys * VW; e += kF32Threads) {
      const int r = kNCHW ? e % kF32Keys : e / VW;
      const int d = kNCHW ? e / kF32Keys : e % VW;
      vs[r][d] = m0 + r < a.n_k ? a.v[vi(m0 + r, d)] : 0.0f;
    }
    __syncthreads();
    // This lane's keys of the tile, lane + 4u: independent dot products, then
    // one rescale of O and the row sum by the new maximum, then P times V.
    const int cnt = min(kF32Keys, a.n_k - m0);
    float sc[kF32Sub];
    float mt = m;
#pragma unroll
    for (int u = 0; u < kF32Sub; ++u) {
      const int r = lane + kF32Lanes * u;
      float s = 0.0f;
#pragma unroll
      for (int d = 0; d < KD; ++d) s = fmaf(q[d], ks[r][d], s);
      sc[u] = r < cnt ? s * a.scale : -INFINITY;   // keys past n_k: P = 0
      mt = fmaxf(mt, sc[u]);
    }
    if (mt == -INFINITY) continue;       // no key of this lane yet
    const float alpha = expf(m - mt);    // 0 while m = -inf
    l *= alpha;
#pragma unroll
    for (int d = 0; d < VW; ++d) o[d] *= alpha;
#pragma unroll
    for (int u = 0; u < kF32Sub; ++u) {
      const float p = expf(sc[u] - mt);
      l += p;
#pragma unroll
      for (int d = 0; d < VW; ++d) o[d] = fmaf(p, vs[lane + kF32Lanes * u][d], o[d]);
    }
    m = mt;
  }
  // Combine the row's four partial softmaxes (a lane with no key has m = -inf, l = 0, O = 0).
#pragma unroll
  for (int x = 1; x < kF32Lanes; x <<= 1) {
    const float mo = __shfl_xor(m, x);
    const float lo = __shfl_xor(l, x);
    const float mn = fmaxf(m, mo);
    const float a0 = m == -INFINITY ? 0.0f : expf(m - mn);
    const float a1 = mo == -INFINITY ? 0.0f : expf(mo - mn);
    l = l * a0 + lo * a1;
#pragma unroll
    for (int d = 0; d < VW; ++d) o[d] = o[d] * a0 + __shfl_xor(o[d], x) * a1;
    m = mn;
  }
  if (!ok) return;
  const float inv = 1.0f / l;
  auto oi = [&](int d) -> int64_t {
    return kNCHW ? (static_cast<int64_t>(bh) * 2 * KD + j * KD + d) * N + row
                 : (static_cast<int64_t>(bh) * a.n_q + row) * KD + d;
  };
  // Each lane stores the columns d = lane (mod 4).
#pragma unroll
  for (int d = 0; d < VW; ++d) {
    if (d % kF32Lanes != lane) continue;
    a.o[oi(d)] = o[d] * inv;
    if (kNCHW && a.vres != nullptr) a.vres[oi(d)] = a.v[vi(row, d)];
  }
  if (a.lse != nullptr && j == 0 && lane == 0)
    a.lse[static_cast<int64_t>(bh) * a.n_q + row] = m + logf(l);
}

// ------------------------------------------------------------------ dispatch

// Compute units of the current device (0 if unknown). The per-device cache is
// atomic: threads that fill it at the same time all store the same value.
int cu_count() {
  static std::atomic<int> cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0 && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
    cus[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Pieces per tail tile. With `slots` workgroups resident at once, `total`
// query tiles leave rem = total mod slots for a last round. If that round
// would fill at most half the slots, its tiles are cut into
// min(slots / rem, n_tiles / kSplitMinTiles, kMaxSplits) key-range pieces,
// when that is at least 2. Returns 1 (and rem = 0) for no split.
int tail_splits(int total, int slots, int n_tiles, int& rem) {
  rem = 0;
  if (slots <= 0 || total <= slots) return 1;
  const int r = total % slots;
  if (r == 0 || 2 * r > slots) return 1;
  int s = slots / r;
  if (s > n_tiles / kSplitMinTiles) s = n_tiles / kSplitMinTiles;
  if (s > kMaxSplits) s = kMaxSplits;
  if (s < 2) return 1;
  rem = r;
  return s;
}

// Query tiles, split plan and the workspace bytes the split needs for one
// launch of attn_fwd_bf16<KD, DV, kNCHW, kVecN, kWaves, kOcc> on the current device.
constexpr int kMinVresWgs = 64;

struct FwdPlan {
  int q_tiles, full, tail, splits, slots;
  size_t bytes;
};

// Query tiles and split plan for `occ` resident workgroups per CU of BM queries each.
FwdPlan make_plan(int occ, int BM, int part_floats, int BH, int n_q, int n_k) {
  FwdPlan p;
  p.q_tiles = (n_q + BM - 1) / BM;
  const int total = BH * p.q_tiles;
  int rem = 0;
  p.slots = occ * cu_count();
  p.splits = tail_splits(total, p.slots, (n_k + kBN - 1) / kBN, rem);
  p.tail = rem;
  p.full = total - rem;
  p.bytes = sizeof(float) * static_cast<size_t>(part_floats) * rem * p.splits;
  return p;
}

// Resident workgroups per CU of a kernel (the same on every gfx950), cached
// atomically per kernel: threads that fill a cache at the same time all store
// the same value.
template <typename K>
int occupancy(K kernel, int threads, std::atomic<int>& cache) {
  int occ = cache.load(std::memory_order_relaxed);
  if (occ < 0) {
    int n = 0;
    occ = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(kernel), threads, 0) ==
                  hipSuccess ? n : 0;
    cache.store(occ, std::memory_order_relaxed);
  }
  return occ;
}

template <int KD, int DV, bool kNCHW, bool kVecN, int kWaves, int kOcc>
FwdPlan plan_bf16(int BH, int n_q, int n_k) {
  using C = FwdCfg<KD, DV, kNCHW, kWaves, direct_staging<KD, kNCHW, kVecN>()>;
  static std::atomic<int> occ_cache{-1};
  const int occ = occupancy(attn_fwd_bf16<KD, DV, kNCHW, kVecN, kWaves, kOcc>, C::NT, occ_cache);
  return make_plan(occ, C::BM, C::PART, BH, n_q, n_k);
}

// Sets the launch fields of `a` from plan p (splitting the tail only if `ws`
// holds the plan's bytes) and returns the number of attention workgroups.
int apply_plan(FwdArgs& a, FwdPlan& p, void* ws, size_t ws_bytes, bool vres_wgs_ok) {
  if (p.tail > 0 && (ws == nullptr || ws_bytes < p.bytes)) {
    p.full += p.tail;
    p.tail = 0;
    p.splits = 1;
  }
  a.q_tiles = p.q_tiles;
  a.full = p.full;
  a.tail = p.tail;
  a.splits = p.splits;
  a.part = static_cast<float*>(ws);
  // When the tail is split, its pieces leave HBM mostly idle: the V residual
  // then goes to extra workgroups on the slots the last round leaves free (at
  // least kMinVresWgs of them). Otherwise each workgroup copies its own
  // pixels' V channels before its key loop (copy workgroups beside a last
  // round of whole query tiles measured slower).
  const int n_attn = p.full + p.tail * p.splits;
  a.vres_wgs = 0;
  if (vres_wgs_ok && a.vres != nullptr && p.tail > 0 && p.slots > 0) {
    const int last = n_attn % p.slots;
    if (last != 0 && p.slots - last >= kMinVresWgs) a.vres_wgs = p.slots - last;
  }
  return n_attn;
}

// Launches the forward; splits the tail only if `ws` holds the plan's bytes.
template <int KD, int DV, bool kNCHW, bool kVecN, int kWaves, int kOcc>
hipError_t launch_bf16(FwdArgs a, void* ws, size_t ws_bytes, hipStream_t stream) {
  using C = FwdCfg<KD, DV, kNCHW, kWaves, direct_staging<KD, kNCHW, kVecN>()>;
  FwdPlan p = plan_bf16<KD, DV, kNCHW, kVecN, kWaves, kOcc>(a.BH, a.n_q, a.n_k);
  const int n_attn = apply_plan(a, p, ws, ws_bytes, kNCHW && kVecN);
  attn_fwd_bf16<KD, DV, kNCHW, kVecN, kWaves, kOcc>
      <<<dim3(static_cast<unsigned>(n_attn + a.vres_wgs)), C::NT, 0, stream>>>(a);
  if (p.tail > 0) {
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    constexpr int chunks = DV / (kMergeThreads / (C::BM / 4));
    attn_fwd_merge<DV, kNCHW, C::BM, C::PART>
        <<<dim3(static_cast<unsigned>(p.tail * chunks)), kMergeThreads, 0, stream>>>(a);
  }
  return hipGetLastError();
}

// Workgroups per CU the registers must allow for head dims up to 64: four for
// directly staged NCHW tiles at key_dim 32 (whose 24 KB of LDS allow four;
// the two-tile loop would otherwise take 130 VGPRs), three for them at key_dim
// 64 (48 KB of LDS), else two. Head dim 128: two for fa2_fwd (220 VGPRs, no spills; with no cap
// the compiler took 296 and ran one), one for the fused kernel (value width
// 256 needs more than half the register file).
template <int KD, bool kNCHW, bool kVecN>
constexpr int occ_target() {
  return KD > 64 ? (kNCHW ? 1 : 2) : (kNCHW && kVecN && KD == 64) ? 3 : (kNCHW && kVecN && KD == 32) ? 4 : 2;
}

// NCHW tiles are staged straight into LDS with buffer loads whose offsets
// (32-bit) span one batch-head's [4*KD][N] slab: N a multiple of 8 and the
// slab under 2 GB. Other maps pass through registers.
// Packed K and V rows are staged straight into LDS with buffer loads whose
// offsets (32-bit) span one batch-head's [n_k][D] rows: under 2 GB.
bool packed_direct(int n_k, int D) {
  return static_cast<int64_t>(n_k) * D * 2 < (int64_t(1) << 31);
}

bool fused_direct(int KD, int N) {
  return N % 8 == 0 && static_cast<int64_t>(8) * KD * N < (int64_t(1) << 31);
}

template <int KD, int DV, bool kNCHW>
hipError_t run_bf16(FwdArgs a, bool vec_n, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (vec_n)
    return launch_bf16<KD, DV, kNCHW, true, kWavesFwd, occ_target<KD, kNCHW, true>()>(a, ws, ws_bytes, stream);
  return launch_bf16<KD, DV, kNCHW, false, kWavesFwd, occ_target<KD, kNCHW, false>()>(a, ws, ws_bytes, stream);
}

template <int KD, int DV, bool kNCHW>
size_t split_bytes(int BH, int n_q, int n_k, bool vec_n) {
  if (vec_n) return plan_bf16<KD, DV, kNCHW, true, kWavesFwd, occ_target<KD, kNCHW, true>()>(BH, n_q, n_k).bytes;
  return plan_bf16<KD, DV, kNCHW, false, kWavesFwd, occ_target<KD, kNCHW, false>()>(BH, n_q, n_k).bytes;
}

template <int KD, bool kNCHW>
hipError_t run_f32(FwdArgsF32 a, hipStream_t stream) {
  const int64_t per_bh = static_cast<int64_t>((a.n_q + kF32Rows - 1) / kF32Rows) * f32_parts<KD, kNCHW>();
  // A launch holds at most 2^31 work-items: batch-heads in as many launches as that takes.
  const int64_t max_bh = std::max<int64_t>(1, (int64_t(1) << 31) / (per_bh * kF32Threads));
  for (int64_t b0 = 0; b0 < a.BH; b0 += max_bh) {
    FwdArgsF32 c = a;
    c.bh0 = static_cast<int>(b0);
    const int64_t nb = std::min<int64_t>(max_bh, a.BH - b0);
    attn_fwd_f32<KD, kNCHW><<<dim3(static_cast<unsigned>(per_bh * nb)), kF32Threads, 0, stream>>>(c);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

size_t fa2_fwd_split_bytes(int BH, int n_q, int n_k, int D, bool bf16) {
  if (!bf16) return 0;
  switch (D) {
    case 16: return split_bytes<16, 16, false>(BH, n_q, n_k, packed_direct(n_k, 16));
    case 32: return split_bytes<32, 32, false>(BH, n_q, n_k, packed_direct(n_k, 32));
    case 64: return split_bytes<64, 64, false>(BH, n_q, n_k, packed_direct(n_k, 64));
    case 128: return split_bytes<128, 128, false>(BH, n_q, n_k, packed_direct(n_k, 128));
  }
  return 0;
}

size_t psa_fused_split_bytes(int BH, int KD, int N, bool bf16) {
  if (!bf16) return 0;
  const bool vec_n = fused_direct(KD, N);
  switch (KD) {
    case 16: return split_bytes<16, 32, true>(BH, N, N, vec_n);
    case 32: return split_bytes<32, 64, true>(BH, N, N, vec_n);
    case 64: return split_bytes<64, 128, true>(BH, N, N, vec_n);
    case 128: return split_bytes<128, 256, true>(BH, N, N, vec_n);
  }
  return 0;
}

hipError_t launch_fa2_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int BH,
                          int n_q, int n_k, int D, float scale, bool bf16, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
  if (!bf16) {
    FwdArgsF32 a{static_cast<const float*>(q), static_cast<const float*>(k),
                 static_cast<const float*>(v), static_cast<float*>(o), nullptr, lse, BH, n_q, n_k,
                 scale};
    switch (D) {
      case 16: return run_f32<16, false>(a, stream);
      case 32: return run_f32<32, false>(a, stream);
      case 64: return run_f32<64, false>(a, stream);
      case 128: return run_f32<128, false>(a, stream);
    }
    return hipErrorInvalidValue;
  }
  FwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.BH = BH;
  a.n_q = n_q;
  a.n_k = n_k;
  a.c = scale * kLog2e;
  switch (D) {
    case 16: return run_bf16<16, 16, false>(a, packed_direct(n_k, 16), ws, ws_bytes, stream);
    case 32: return run_bf16<32, 32, false>(a, packed_direct(n_k, 32), ws, ws_bytes, stream);
    case 64: return run_bf16<64, 64, false>(a, packed_direct(n_k, 64), ws, ws_bytes, stream);
    case 128: return run_bf16<128, 128, false>(a, packed_direct(n_k, 128), ws, ws_bytes, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_psa_fused_fwd(const void* qkv, void* out, void* vres, float* lse, int BH, int KD,
                                int N, float scale, bool bf16, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
  if (!bf16) {
    const float* x = static_cast<const float*>(qkv);
    FwdArgsF32 a{x, x, x, static_cast<float*>(out), static_cast<float*>(vres), lse, BH, N, N, scale};
    switch (KD) {
      case 16: return run_f32<16, true>(a, stream);
      case 32: return run_f32<32, true>(a, stream);
      case 64: return run_f32<64, true>(a, stream);
      case 128: return run_f32<128, true>(a, stream);
    }
    return hipErrorInvalidValue;
  }
  const uint16_t* x = static_cast<const uint16_t*>(qkv);
  FwdArgs a{};
  a.q = x;
  a.k = x;
  a.v = x;
  a.o = static_cast<uint16_t*>(out);
  a.vres = static_cast<uint16_t*>(vres);
  a.lse = lse;
  a.BH = BH;
  a.n_q = N;
  a.n_k = N;
  a.c = scale * kLog2e;
  const bool vec_n = fused_direct(KD, N);
  switch (KD) {
    case 16: return run_bf16<16, 32, true>(a, vec_n, ws, ws_bytes, stream);
    case 32: return run_bf16<32, 64, true>(a, vec_n, ws, ws_bytes, stream);
    case 64: return run_bf16<64, 128, true>(a, vec_n, ws, ws_bytes, stream);
    case 128: return run_bf16<128, 256, true>(a, vec_n, ws, ws_bytes, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace psa
