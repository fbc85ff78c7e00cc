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
// queries and walks all keys in tiles of 64, staged in LDS by plain 16-byte
// copies in the tensors' own layout (double-buffered: the next tile's global
// loads are in flight while the current tile is computed).
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

#include "psa_device.hpp"
#include "psa_launch.hpp"

namespace psa {
namespace {

constexpr int kBN = 64;   // keys per tile
constexpr int kPad = 8;   // bf16 elements of padding per LDS row (spreads banks)

#ifndef PSA_LAZY_RESCALE
#define PSA_LAZY_RESCALE 1
#endif

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

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
};

// blockIdx -> (bh, query tile). Workgroups are dispatched round-robin over the
// 8 XCDs; this remap gives each XCD a contiguous run of logical tiles, so the
// query tiles of one batch-head share an L2 and its K/V stay resident there.
__device__ __forceinline__ void tile_of_block(int total, int q_tiles, int& bh, int& qt) {
  const int i = blockIdx.x;
  const int per = total / 8;
  const int L = (i < per * 8) ? (i % 8) * per + i / 8 : i;
  bh = L / q_tiles;
  qt = L - bh * q_tiles;
}

__device__ __forceinline__ u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

__device__ __forceinline__ u32x4 load16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// 8 bf16 values p[0], p[stride], ..., p[7*stride], zero where idx0 + e >= limit.
__device__ __forceinline__ u32x4 gather8(const uint16_t* p, int64_t stride, int idx0, int limit) {
  u32x4 r;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t lo = (idx0 + 2 * w < limit) ? p[(2 * w) * stride] : 0u;
    const uint32_t hi = (idx0 + 2 * w + 1 < limit) ? p[(2 * w + 1) * stride] : 0u;
    r[w] = lo | (hi << 16);
  }
  return r;
}

// Two ds_read_b64_tr_b16 (rows p[0..3] and p[4*row..]) forming one 8-value operand.
__device__ __forceinline__ bf16x8 lds_read_tr8(const uint16_t* p, int row) {
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p + 4 * row));
  const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
  return as_bf16x8(u32x4{a[0], a[1], b[0], b[1]});
}

#ifndef PSA_USE_PERMLANE
#define PSA_USE_PERMLANE 1
#endif
// Value of x held by lane ^ 32 (g = lane / 32).
__device__ __forceinline__ float lane_xor32(float x, int g) {
#if PSA_USE_PERMLANE
  const u32x2 sw = __builtin_bit_cast(u32x2, __builtin_amdgcn_permlane32_swap(
      __builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x), false, false));
  return __builtin_bit_cast(float, g ? sw[0] : sw[1]);
#else
  (void)g;
  return __shfl_xor(x, 32);
#endif
}

// Key held by S^T row rho (0..31) of a 32-key block: 8h + 4g + e -> 8g + 4h + e
// inside each 16-row half.
__device__ __forceinline__ int key_of_row(int rho) {
  return (rho & 16) | ((rho & 4) << 1) | ((rho & 8) >> 1) | (rho & 3);
}

// Column offset (in keys) a 16-lane group's source lane s supplies for the
// transposed K read, so that output lane i receives key key_of_row(i).
__device__ __forceinline__ int tr_key_col(int s) { return ((s & 1) << 3) | ((s & 2) << 1); }

template <int KD, int DV, bool kNCHW, int kWaves, int kQB, bool kDirect = false>
struct FwdCfg {
  static constexpr int NT = kWaves * 64;
  static constexpr int BM = 32 * kQB * kWaves;   // queries per workgroup
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
};

// Position of 16-byte chunk c (8 keys) of V row dv in the unpadded, directly
// staged V tile: an XOR swizzle that puts the 16 rows read together by one
// 16-byte-per-lane instruction on 16 different bank groups.
__device__ __forceinline__ int v_chunk_pos(int dv, int c) { return c ^ ((dv >> 1) & 7); }

// Direct global -> LDS staging of one NCHW key tile (N a multiple of 8): each
// wave instruction (global_load_lds_dwordx4) fills 64 consecutive 16-byte LDS
// chunks, lane i the i-th; lanes pick which global chunk to fetch, which is
// how the V swizzle is applied. No registers and no LDS write instructions;
// the wave waits with vmcnt before the barrier that publishes the tile.
template <int KD, int DV, int kWaves>
struct FwdStageDirect {
  static constexpr int K_BLOCKS = KD * (kBN / 8) / 64;     // 1 KB blocks of K
  static constexpr int V_BLOCKS = DV * (kBN / 8) / 64;     // 1 KB blocks of V
  static constexpr int BLOCKS = K_BLOCKS + V_BLOCKS;
  static_assert(KD * (kBN / 8) % 64 == 0 && DV * (kBN / 8) % 64 == 0, "whole 1 KB blocks");

  __device__ __forceinline__ void issue(const FwdArgs& a, int bh, int kt, int wave, int lane,
                                        uint16_t* buf) const {
    const int N = a.n_k;
    const int m0 = kt * kBN;
#pragma unroll
    for (int i = 0; i < (BLOCKS + kWaves - 1) / kWaves; ++i) {
      const int b = wave + i * kWaves;
      if (b >= BLOCKS) break;
      const int p = b * 64 + lane;                 // LDS chunk this lane fills
      const bool is_k = b < K_BLOCKS;
      const int q = is_k ? p : p - K_BLOCKS * 64;
      const int row = q >> 3;                      // d (K) or dv (V)
      const int c = is_k ? (q & 7) : v_chunk_pos(row, q & 7);
      int m = m0 + c * 8;
      m = m < N ? m : N - 8;                       // keys past n_k: real data, masked later
      const int64_t ch = static_cast<int64_t>(bh) * 4 * KD + (is_k ? KD : 2 * KD) + row;
      __builtin_amdgcn_global_load_lds(a.k + ch * N + m,
                                       (__attribute__((address_space(3))) void*)(buf + b * 512), 16, 0, 0);
    }
  }
};

// Global -> registers -> LDS staging of one key tile (K and V), 16-byte chunks.
// Keys past n_k are clamped to real rows (finite data): their scores are
// masked to -inf, so they contribute nothing. The unaligned NCHW variant
// (N not a multiple of 8) gathers element by element and zero-fills instead.
template <int KD, int DV, bool kNCHW, bool kVecN, int kWaves, int kQB>
struct FwdStage {
  using C = FwdCfg<KD, DV, kNCHW, kWaves, kQB>;
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

// kQB: 32-query blocks per wave. With two, every K and V operand read from LDS
// feeds two MFMAs (the LDS traffic per flop halves) and the two softmax chains
// are independent work the wave interleaves with its MFMAs.
// kOcc: waves per SIMD the register allocation must allow.
template <int KD, int DV, bool kNCHW, bool kVecN, int kWaves, int kQB, int kOcc>
__global__ __launch_bounds__(kWaves * 64, kOcc) void attn_fwd_bf16(FwdArgs a) {
  constexpr bool kDirect = kNCHW && kVecN;   // direct global -> LDS staging
  using C = FwdCfg<KD, DV, kNCHW, kWaves, kQB, kDirect>;
  constexpr int NT = C::NT;
  constexpr int BM = C::BM;
  constexpr int NKB = kBN / 32;        // 32-key blocks per tile
  constexpr int NKS = kBN / 16;        // 16-key MFMA steps per tile
  constexpr int NDS = KD / 16;         // 16-wide d steps of K Q^T
  constexpr int NDB = C::DVP / 32;     // 32-row blocks of O^T
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * C::BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int g = lane >> 5;           // lane group of the MFMA layouts
  const int i16 = lane & 15;         // lane inside its 16-lane group
  const int t16 = (lane >> 4) & 1;   // which 16-row half of an operand block
  int bh, qt;
  tile_of_block(a.BH * a.q_tiles, a.q_tiles, bh, qt);
  const int N = a.n_k;   // NCHW: n_q == n_k == H*W
  int q_row[kQB];
  bool q_ok[kQB];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    q_row[qb] = qt * BM + (wave * kQB + qb) * 32 + l32;
    q_ok[qb] = q_row[qb] < a.n_q;
  }

  // Packed V with DV = 16: columns 16..31 of every V row stay zero in both buffers.
  if constexpr (!kNCHW && C::DVP > DV) {
    for (int e = tid; e < kBN * (C::DVP - DV); e += NT) {
      const int row = e / (C::DVP - DV), col = DV + e % (C::DVP - DV);
      smem[C::K_ELEMS + row * C::VROW + col] = 0;
      smem[C::BUF + C::K_ELEMS + row * C::VROW + col] = 0;
    }
  }

  // V residual: copy this tile's pixel columns of the V channels (NCHW only).
  if constexpr (kNCHW) {
    if (a.vres != nullptr) {
      const int n0 = qt * BM;
      constexpr int CPR = BM / 8;   // 8-pixel chunks per channel row
      for (int c = tid; c < DV * CPR; c += NT) {
        const int dv = c / CPR, cb = c % CPR;
        const int n = n0 + cb * 8;
        const uint16_t* src = a.v + (static_cast<int64_t>(bh) * 4 * KD + 2 * KD + dv) * N + n;
        uint16_t* dst = a.vres + (static_cast<int64_t>(bh) * DV + dv) * N + n;
        if constexpr (kVecN) {
          if (n < N) stg_nt(reinterpret_cast<u32x4*>(dst), load16(src));
        } else {
          for (int e = 0; e < 8; ++e)
            if (n + e < N) dst[e] = src[e];
        }
      }
    }
  }

  // This lane's Q operands: Q[q_row][16*ds + 8*g + j], j = 0..7.
  bf16x8 qop[kQB][NDS];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      u32x4 raw = zero4();
      if (q_ok[qb]) {
        if constexpr (kNCHW) {
          const uint16_t* src = a.q + (static_cast<int64_t>(bh) * 4 * KD + ds * 16 + g * 8) * N + q_row[qb];
          raw = gather8(src, N, 0, 8);
        } else {
          raw = load16(a.q + (static_cast<int64_t>(bh) * a.n_q + q_row[qb]) * KD + ds * 16 + g * 8);
        }
      }
      qop[qb][ds] = as_bf16x8(raw);
    }

  f32x16 oacc[kQB][NDB];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[qb][db][r] = 0.0f;
  float m_run[kQB], l_run[kQB];   // running max of scale*log2(e)*S; this lane's part of the sum
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.0f;
  }

  const int n_tiles = (a.n_k + kBN - 1) / kBN;
  FwdStage<KD, DV, kNCHW, kVecN, kWaves, kQB> stage;
  FwdStageDirect<KD, DV, kWaves> dstage;
  if constexpr (kDirect) {
    dstage.issue(a, bh, 0, wave, lane, smem);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  } else {
    stage.load(a, bh, 0, tid);
    stage.store(smem, tid);
  }
  __syncthreads();

  for (int kt = 0; kt < n_tiles; ++kt) {
    const uint16_t* ks = smem + (kt & 1) * C::BUF;
    const uint16_t* vs = ks + C::K_ELEMS;
    const bool more = kt + 1 < n_tiles;
    if constexpr (kDirect) {
      if (more) dstage.issue(a, bh, kt + 1, wave, lane, smem + ((kt + 1) & 1) * C::BUF);
    } else {
      if (more) stage.load(a, bh, kt + 1, tid);
    }

    // S^T = K Q^T for the tile's keys (rows permuted by key_of_row); one K
    // operand read serves every query block.
    f32x16 sacc[kQB][NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[qb][kb][r] = 0.0f;
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        bf16x8 kop;
        if constexpr (kNCHW)
          kop = lds_read_tr8(ks + (ds * 16 + 8 * g + (i16 >> 2)) * C::KROW + kb * 32 + 16 * t16 +
                                 tr_key_col(i16 & 3), C::KROW);
        else
          kop = *reinterpret_cast<const bf16x8*>(ks + (kb * 32 + key_of_row(l32)) * C::KROW + ds * 16 + g * 8);
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) sacc[qb][kb] = mfma32x32x16(kop, qop[qb][ds], sacc[qb][kb]);
      }
    }
    // Keys past n_k (last tile only) get -inf. Element r of block kb holds
    // key 32*kb + 16*(r/8) + 8*g + r%8 of the tile.
    if ((kt + 1) * kBN > a.n_k) {
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kt * kBN + kb * 32 + 16 * (r >> 3) + 8 * g + (r & 7);
            if (key >= a.n_k) sacc[qb][kb][r] = -INFINITY;
          }
    }

    // Online softmax per query block: running max, rescale, P = 2^(c*S - m).
    bf16x8 pop[kQB][NKS];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      float mx = sacc[qb][0][0];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[qb][kb][r]);
      mx = fmaxf(mx, lane_xor32(mx, g));
      const float m_tile = mx * a.c;
#if PSA_LAZY_RESCALE
      // The running max only moves when some lane's tile max exceeds it by
      // more than 8 (log2 units): until then P <= 2^8, harmless in fp32 and bf16.
      if (__any(m_tile > m_run[qb] + 8.0f)) {
#else
      {
#endif
        const float m_new = fmaxf(m_run[qb], m_tile);
        const float alpha = fast_exp2(m_run[qb] - m_new);
        m_run[qb] = m_new;
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[qb][db][r] *= alpha;
      }
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          pop[qb][s][j] = static_cast<__bf16>(fast_exp2(fmaf(sacc[qb][s >> 1][8 * (s & 1) + j], a.c, -m_run[qb])));
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          const bf16x2 pp = {pop[qb][s][j], pop[qb][s][j + 1]};
          l_run[qb] = __builtin_amdgcn_fdot2_f32_bf16(pp, bf16x2{1.0f, 1.0f}, l_run[qb], false);
        }
      }
    }

    // O^T += V^T P^T: step s covers keys 16s + 8g + j of the tile in this lane's P;
    // one V operand read serves every query block.
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        bf16x8 vop;
        if constexpr (kDirect)
          vop = *reinterpret_cast<const bf16x8*>(vs + (db * 32 + l32) * C::VROW +
                                                 v_chunk_pos(db * 32 + l32, 2 * s + g) * 8);
        else if constexpr (kNCHW)
          vop = *reinterpret_cast<const bf16x8*>(vs + (db * 32 + l32) * C::VROW + s * 16 + g * 8);
        else
          vop = lds_read_tr8(vs + (s * 16 + 8 * g + (i16 >> 2)) * C::VROW + db * 32 + 16 * t16 + 4 * (i16 & 3),
                             C::VROW);
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) oacc[qb][db] = mfma32x32x16(vop, pop[qb][s], oacc[qb][db]);
      }

    if constexpr (kDirect) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's part of tile kt+1 landed
    } else {
      if (more) stage.store(smem + ((kt + 1) & 1) * C::BUF, tid);
    }
    __syncthreads();
  }

  // Epilogue: O = O^T / l, LSE = (m + log2 l) ln 2.
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const float l_tot = l_run[qb] + lane_xor32(l_run[qb], g);
    const float inv = 1.0f / l_tot;
    if (!q_ok[qb]) continue;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int dv0 = db * 32 + 8 * r4 + 4 * g;   // rows dv0 .. dv0+3 of this lane
        if (dv0 >= DV) continue;
        uint16_t h[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = float_to_bf16_bits(oacc[qb][db][4 * r4 + e] * inv);
        if constexpr (kNCHW) {
          uint16_t* dst = a.o + (static_cast<int64_t>(bh) * DV + dv0) * N + q_row[qb];
#pragma unroll
          for (int e = 0; e < 4; ++e) dst[static_cast<int64_t>(e) * N] = h[e];
        } else {
          uint16_t* dst = a.o + (static_cast<int64_t>(bh) * a.n_q + q_row[qb]) * DV + dv0;
          *reinterpret_cast<u32x2*>(dst) = u32x2{h[0] | (uint32_t(h[1]) << 16), h[2] | (uint32_t(h[3]) << 16)};
        }
      }
    if (a.lse != nullptr && g == 0)
      a.lse[static_cast<int64_t>(bh) * a.n_q + q_row[qb]] = (m_run[qb] + log2f(l_tot)) * kLn2;
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
};

constexpr int kF32Threads = 128;
constexpr int kF32Keys = 32;

// One thread per query row, keys staged through LDS in tiles of 32, float32
// throughout with expf. Workgroups enumerate (bh, V half, query block); the
// fused (NCHW) variant has two V halves, the packed variant one.
template <int KD, bool kNCHW>
__global__ __launch_bounds__(kF32Threads) void attn_fwd_f32(FwdArgsF32 a) {
  __shared__ float ks[kF32Keys][KD];
  __shared__ float vs[kF32Keys][KD];
  const int halves = kNCHW ? 2 : 1;
  const int q_blocks = (a.n_q + kF32Threads - 1) / kF32Threads;
  const int qb = blockIdx.x % q_blocks;
  const int bh = (blockIdx.x / q_blocks) / halves;
  const int j = (blockIdx.x / q_blocks) % halves;
  const int row = qb * kF32Threads + threadIdx.x;
  const bool ok = row < a.n_q;
  const int N = a.n_k;
  // Element (row n, column d) of Q, K and V half j, in either layout.
  auto qi = [&](int n, int d) -> int64_t {
    return kNCHW ? (static_cast<int64_t>(bh) * 4 * KD + d) * N + n
                 : (static_cast<int64_t>(bh) * a.n_q + n) * KD + d;
  };
  auto ki = [&](int n, int d) -> int64_t {
    return kNCHW ? (static_cast<int64_t>(bh) * 4 * KD + KD + d) * N + n
                 : (static_cast<int64_t>(bh) * a.n_k + n) * KD + d;
  };
  auto vi = [&](int n, int d) -> int64_t {
    return kNCHW ? (static_cast<int64_t>(bh) * 4 * KD + (2 + j) * KD + d) * N + n
                 : (static_cast<int64_t>(bh) * a.n_k + n) * KD + d;
  };
  float q[KD], o[KD];
#pragma unroll
  for (int d = 0; d < KD; ++d) {
    q[d] = ok ? a.q[qi(row, d)] : 0.0f;
    o[d] = 0.0f;
  }
  float m = -INFINITY, l = 0.0f;
  for (int m0 = 0; m0 < a.n_k; m0 += kF32Keys) {
    __syncthreads();
    for (int e = threadIdx.x; e < kF32Keys * KD; e += kF32Threads) {
      const int r = kNCHW ? e % kF32Keys : e / KD;
      const int d = kNCHW ? e / kF32Keys : e % KD;
      const bool in = m0 + r < a.n_k;
      ks[r][d] = in ? a.k[ki(m0 + r, d)] : 0.0f;
      vs[r][d] = in ? a.v[vi(m0 + r, d)] : 0.0f;
    }
    __syncthreads();
    const int cnt = min(kF32Keys, a.n_k - m0);
    for (int r = 0; r < cnt; ++r) {
      float s = 0.0f;
#pragma unroll
      for (int d = 0; d < KD; ++d) s = fmaf(q[d], ks[r][d], s);
      s *= a.scale;
      const float m_new = fmaxf(m, s);
      const float alpha = expf(m - m_new);
      const float p = expf(s - m_new);
      l = l * alpha + p;
#pragma unroll
      for (int d = 0; d < KD; ++d) o[d] = fmaf(p, vs[r][d], o[d] * alpha);
      m = m_new;
    }
  }
  if (!ok) return;
  const float inv = 1.0f / l;
#pragma unroll
  for (int d = 0; d < KD; ++d) {
    const int64_t oi = kNCHW ? (static_cast<int64_t>(bh) * 2 * KD + j * KD + d) * N + row
                             : (static_cast<int64_t>(bh) * a.n_q + row) * KD + d;
    a.o[oi] = o[d] * inv;
    if (kNCHW && a.vres != nullptr) a.vres[oi] = a.v[vi(row, d)];
  }
  if (a.lse != nullptr && j == 0) a.lse[static_cast<int64_t>(bh) * a.n_q + row] = m + logf(l);
}

// ------------------------------------------------------------------ dispatch

#ifndef PSA_QB
#define PSA_QB 1
#endif

template <int KD, int DV, bool kNCHW, int kWaves>
hipError_t run_bf16(FwdArgs a, bool vec_n, hipStream_t stream) {
  // Two 32-query blocks per wave (one wave per SIMD) where the registers allow;
  // head dim 128 keeps one block per wave.
  constexpr int kQB = KD <= 64 ? PSA_QB : 1;
  constexpr int BM = 32 * kQB * kWaves;
#ifdef PSA_FWD_OCC
  constexpr int kOcc = KD <= 64 ? PSA_FWD_OCC : 1;
#else
  constexpr int kOcc = (kQB == 1 && KD <= 64 && 2 * 2 * FwdCfg<KD, DV, kNCHW, kWaves, kQB>::BUF * 2 <= 160 * 1024) ? 2 : 1;
#endif
  a.q_tiles = (a.n_q + BM - 1) / BM;
  const dim3 grid(static_cast<unsigned>(a.BH) * a.q_tiles);
  if (vec_n)
    attn_fwd_bf16<KD, DV, kNCHW, true, kWaves, kQB, kOcc><<<grid, kWaves * 64, 0, stream>>>(a);
  else
    attn_fwd_bf16<KD, DV, kNCHW, false, kWaves, kQB, kOcc><<<grid, kWaves * 64, 0, stream>>>(a);
  return hipGetLastError();
}

template <int KD, bool kNCHW>
hipError_t run_f32(FwdArgsF32 a, hipStream_t stream) {
  const unsigned q_blocks = (a.n_q + kF32Threads - 1) / kF32Threads;
  const dim3 grid(q_blocks * a.BH * (kNCHW ? 2 : 1));
  attn_fwd_f32<KD, kNCHW><<<grid, kF32Threads, 0, stream>>>(a);
  return hipGetLastError();
}

#ifndef PSA_FWD_WAVES
#define PSA_FWD_WAVES 4
#endif
constexpr int kWavesFwd = PSA_FWD_WAVES;

}  // namespace

hipError_t launch_fa2_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int BH,
                          int n_q, int n_k, int D, float scale, bool bf16, hipStream_t stream) {
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
  FwdArgs a{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
            static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), nullptr, lse, BH, n_q, n_k,
            0, scale * kLog2e};
  switch (D) {
    case 16: return run_bf16<16, 16, false, kWavesFwd>(a, true, stream);
    case 32: return run_bf16<32, 32, false, kWavesFwd>(a, true, stream);
    case 64: return run_bf16<64, 64, false, kWavesFwd>(a, true, stream);
    case 128: return run_bf16<128, 128, false, kWavesFwd>(a, true, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_psa_fused_fwd(const void* qkv, void* out, void* vres, float* lse, int BH, int KD,
                                int N, float scale, bool bf16, hipStream_t stream) {
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
  FwdArgs a{x, x, x, static_cast<uint16_t*>(out), static_cast<uint16_t*>(vres), lse, BH, N, N, 0,
            scale * kLog2e};
  const bool vec_n = (N % 8) == 0;
  switch (KD) {
    case 16: return run_bf16<16, 32, true, kWavesFwd>(a, vec_n, stream);
    case 32: return run_bf16<32, 64, true, kWavesFwd>(a, vec_n, stream);
    case 64: return run_bf16<64, 128, true, kWavesFwd>(a, vec_n, stream);
    case 128: return run_bf16<128, 256, true, kWavesFwd>(a, vec_n, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace psa
