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
// queries and walks all keys in tiles of 64 staged in LDS (double-buffered,
// the next tile's global loads in flight while the current one is computed).
//
// Per wave and key tile, on the matrix cores (v_mfma_f32_32x32x16_bf16):
//   S^T[key][query] = K Q^T      A = K rows from LDS, B = Q (registers)
//   O^T[dv][query] += V^T P^T    A = V^T rows from LDS, B = P (registers)
// Computing the transposed products puts one query per lane column, so the
// running max and sum are per-lane scalars (one cross-lane step, lane ^ 32),
// and the accumulator layout of S^T is exactly the B-operand layout P needs
// for the second product: P never leaves registers. V^T is stored in LDS with
// keys permuted inside each group of 16 so that a lane's 8 keys are one
// 16-byte read.
//
// Input layouts: "packed" ([BH, n, D] q/k/v, the layout PsaPackQkv writes) or
// "NCHW" (the QKV conv output itself: Q, K, V channel rows of N pixels, so K
// is transposed on its way into LDS and V is not). Softmax runs in base 2
// with scale*log2(e) folded into one multiply-add; P is rounded to bf16 for
// the PV product and the row sum adds the same rounded values.
#include <math.h>

#include "psa_device.hpp"
#include "psa_launch.hpp"

namespace psa {
namespace {

constexpr int kBN = 64;   // keys per tile
constexpr int kPad = 8;   // bf16 elements of padding per LDS row (breaks bank conflicts)

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

// 8x8 transpose of 16-bit elements held as 8 rows of 16 bytes.
__device__ __forceinline__ void transpose8x8(const u32x4 (&in)[8], u32x4 (&out)[8]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t lo = in[2 * w][c >> 1];
      const uint32_t hi = in[2 * w + 1][c >> 1];
      out[c][w] = (c & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
    }
  }
}

// Writes 8 consecutive keys (8*mb .. 8*mb+7 of the tile) of one V^T row into
// their permuted LDS positions: inside each group of 16 keys, key kappa goes
// to 8*((kappa/4)%2) + 4*(kappa/8) + kappa%4.
__device__ __forceinline__ void store_vt8(uint16_t* vt_row, int mb, u32x4 v) {
  const int base = (mb >> 1) * 16 + (mb & 1) * 4;
  *reinterpret_cast<u32x2*>(vt_row + base) = u32x2{v[0], v[1]};
  *reinterpret_cast<u32x2*>(vt_row + base + 8) = u32x2{v[2], v[3]};
}

template <int KD, int DV, bool kNCHW, bool kVecN, int kWaves>
struct FwdTile {
  static constexpr int NT = kWaves * 64;
  static constexpr int DVP = DV < 32 ? 32 : DV;        // V^T rows (padded to one MFMA block)
  static constexpr int KSTR = KD + kPad;               // LDS row stride of K (keys x d)
  static constexpr int VSTR = kBN + kPad;              // LDS row stride of V^T (dv x keys)
  static constexpr int K_ELEMS = kBN * KSTR;
  static constexpr int V_ELEMS = DVP * VSTR;
  static constexpr int BUF = K_ELEMS + V_ELEMS;
  // Staging work per tile.
  static constexpr int K_CHUNKS = kNCHW ? (KD / 8) * (kBN / 8) : kBN * KD / 8;  // 8x8 blocks or 16B rows
  static constexpr int V_CHUNKS = kNCHW ? DV * kBN / 8 : (kBN / 8) * (DV / 8);  // 16B rows or 8x8 blocks
  static constexpr int K_PER = kNCHW ? 1 : (K_CHUNKS + NT - 1) / NT;
  static constexpr int V_PER = kNCHW ? (V_CHUNKS + NT - 1) / NT : 1;
  static_assert(!kNCHW || K_CHUNKS <= NT, "one K block per thread");
  static_assert(kNCHW || V_CHUNKS <= NT, "one V block per thread");
  static constexpr int KREG = kNCHW ? 8 : K_PER;
  static constexpr int VREG = kNCHW ? V_PER : 8;

  u32x4 kr[KREG];
  u32x4 vr[VREG];

  // Global -> registers for key tile kt.
  __device__ __forceinline__ void load(const FwdArgs& a, int bh, int kt, int tid, int N) {
    const int m0 = kt * kBN;
    if constexpr (kNCHW) {
      // K: 8x8 block (d-block db, key-block mb) of the [KD, N] channel rows.
      if (tid < K_CHUNKS) {
        const int db = tid / (kBN / 8), mb = tid % (kBN / 8);
        const int m = m0 + mb * 8;
        const uint16_t* src = a.k + (static_cast<int64_t>(bh) * 4 * KD + KD + db * 8) * N + m;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          if constexpr (kVecN)
            kr[r] = (m < a.n_k) ? load16(src + static_cast<int64_t>(r) * N) : zero4();
          else
            kr[r] = gather8(src + static_cast<int64_t>(r) * N, 1, m, a.n_k);
        }
      }
      // V: 16-byte runs of 8 keys along one of the DV channel rows.
#pragma unroll
      for (int i = 0; i < V_PER; ++i) {
        const int c = tid + i * NT;
        if (c < V_CHUNKS) {
          const int dv = c / (kBN / 8), mb = c % (kBN / 8);
          const int m = m0 + mb * 8;
          const uint16_t* src = a.v + (static_cast<int64_t>(bh) * 4 * KD + 2 * KD + dv) * N + m;
          if constexpr (kVecN)
            vr[i] = (m < a.n_k) ? load16(src) : zero4();
          else
            vr[i] = gather8(src, 1, m, a.n_k);
        }
      }
    } else {
      // K: 16-byte pieces of key rows.
#pragma unroll
      for (int i = 0; i < K_PER; ++i) {
        const int c = tid + i * NT;
        if (c < K_CHUNKS) {
          const int r = c / (KD / 8), cb = c % (KD / 8);
          const int m = m0 + r;
          kr[i] = (m < a.n_k) ? load16(a.k + (static_cast<int64_t>(bh) * a.n_k + m) * KD + cb * 8)
                              : zero4();
        }
      }
      // V: 8x8 block (key-block mb, dv-block db) of the [n_k, DV] rows.
      if (tid < V_CHUNKS) {
        const int mb = tid / (DV / 8), db = tid % (DV / 8);
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int m = m0 + mb * 8 + r;
          vr[r] = (m < a.n_k) ? load16(a.v + (static_cast<int64_t>(bh) * a.n_k + m) * DV + db * 8)
                              : zero4();
        }
      }
    }
  }

  // Registers -> LDS buffer (K as [key][d], V^T as [dv][permuted key]).
  __device__ __forceinline__ void store(uint16_t* buf, int tid) const {
    uint16_t* ks = buf;
    uint16_t* vt = buf + K_ELEMS;
    if constexpr (kNCHW) {
      if (tid < K_CHUNKS) {
        const int db = tid / (kBN / 8), mb = tid % (kBN / 8);
        u32x4 t[8];
        transpose8x8(kr, t);
#pragma unroll
        for (int c = 0; c < 8; ++c)
          *reinterpret_cast<u32x4*>(ks + (mb * 8 + c) * KSTR + db * 8) = t[c];
      }
#pragma unroll
      for (int i = 0; i < V_PER; ++i) {
        const int c = tid + i * NT;
        if (c < V_CHUNKS) {
          const int dv = c / (kBN / 8), mb = c % (kBN / 8);
          store_vt8(vt + dv * VSTR, mb, vr[i]);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < K_PER; ++i) {
        const int c = tid + i * NT;
        if (c < K_CHUNKS) {
          const int r = c / (KD / 8), cb = c % (KD / 8);
          *reinterpret_cast<u32x4*>(ks + r * KSTR + cb * 8) = kr[i];
        }
      }
      if (tid < V_CHUNKS) {
        const int mb = tid / (DV / 8), db = tid % (DV / 8);
        u32x4 t[8];
        transpose8x8(vr, t);
#pragma unroll
        for (int c = 0; c < 8; ++c) store_vt8(vt + (db * 8 + c) * VSTR, mb, t[c]);
      }
    }
  }
};

template <int KD, int DV, bool kNCHW, bool kVecN, int kWaves>
__global__ __launch_bounds__(kWaves * 64) void attn_fwd_bf16(FwdArgs a) {
  using Tile = FwdTile<KD, DV, kNCHW, kVecN, kWaves>;
  constexpr int NT = Tile::NT;
  constexpr int BM = 32 * kWaves;
  constexpr int DVP = Tile::DVP;
  constexpr int NKB = kBN / 32;      // 32-key blocks per tile
  constexpr int NKS = kBN / 16;      // 16-key MFMA steps per tile
  constexpr int NDS = KD / 16;       // 16-wide d steps of Q K^T
  constexpr int NDB = DVP / 32;      // 32-row blocks of O^T
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * Tile::BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int g = lane >> 5;
  int bh, qt;
  tile_of_block(a.BH * a.q_tiles, a.q_tiles, bh, qt);
  const int N = a.n_k;   // NCHW: n_q == n_k == H*W
  const int q_row = qt * BM + wave * 32 + l32;
  const bool q_ok = q_row < a.n_q;

  // Padded V^T rows (DV = 16) stay zero in both buffers.
  if constexpr (DVP > DV) {
    for (int e = tid; e < (DVP - DV) * Tile::VSTR; e += NT) {
      smem[Tile::K_ELEMS + DV * Tile::VSTR + e] = 0;
      smem[Tile::BUF + Tile::K_ELEMS + DV * Tile::VSTR + e] = 0;
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
  bf16x8 qop[NDS];
#pragma unroll
  for (int ds = 0; ds < NDS; ++ds) {
    u32x4 raw = zero4();
    if (q_ok) {
      if constexpr (kNCHW) {
        const uint16_t* src = a.q + (static_cast<int64_t>(bh) * 4 * KD + ds * 16 + g * 8) * N + q_row;
        raw = gather8(src, N, 0, 8);
      } else {
        raw = load16(a.q + (static_cast<int64_t>(bh) * a.n_q + q_row) * KD + ds * 16 + g * 8);
      }
    }
    qop[ds] = as_bf16x8(raw);
  }

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;
  float m_run = -INFINITY;   // running max of scale*log2(e)*S
  float l_run = 0.0f;        // this lane's part of the running sum (keys of lane group g)

  const int n_tiles = (a.n_k + kBN - 1) / kBN;
  Tile tile;
  tile.load(a, bh, 0, tid, N);
  tile.store(smem, tid);
  __syncthreads();

  for (int kt = 0; kt < n_tiles; ++kt) {
    const uint16_t* ks = smem + (kt & 1) * Tile::BUF;
    const uint16_t* vt = ks + Tile::K_ELEMS;
    const bool more = kt + 1 < n_tiles;
    if (more) tile.load(a, bh, kt + 1, tid, N);

    // S^T = K Q^T for the tile's keys.
    f32x16 sacc[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.0f;
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        const bf16x8 kop = *reinterpret_cast<const bf16x8*>(ks + (kb * 32 + l32) * Tile::KSTR + ds * 16 + g * 8);
        sacc[kb] = mfma32x32x16(kop, qop[ds], sacc[kb]);
      }
    }
    // Keys past n_k (last tile only) get -inf.
    if ((kt + 1) * kBN > a.n_k) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt * kBN + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          if (key >= a.n_k) sacc[kb][r] = -INFINITY;
        }
    }

    // Online softmax: new running max, rescale, P = 2^(c*S - m).
    float mx = sacc[0][0];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * a.c);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;

    bf16x8 pop[NKS];
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float p = fast_exp2(fmaf(sacc[s >> 1][8 * (s & 1) + j], a.c, -m_new));
        pop[s][j] = static_cast<__bf16>(p);
      }
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const bf16x2 pp = {pop[s][j], pop[s][j + 1]};
        l_run = __builtin_amdgcn_fdot2_f32_bf16(pp, bf16x2{1.0f, 1.0f}, l_run, false);
      }
    }

    // O^T += V^T P^T.
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        const bf16x8 vop = *reinterpret_cast<const bf16x8*>(vt + (db * 32 + l32) * Tile::VSTR + s * 16 + g * 8);
        oacc[db] = mfma32x32x16(vop, pop[s], oacc[db]);
      }

    if (more) tile.store(smem + ((kt + 1) & 1) * Tile::BUF, tid);
    __syncthreads();
  }

  // Epilogue: O = O^T / l, LSE = (m + log2 l) ln 2.
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
  if (q_ok) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int dv0 = db * 32 + 8 * r4 + 4 * g;   // rows dv0 .. dv0+3 of this lane
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

template <int KD, int DV, bool kNCHW, int kWaves>
hipError_t run_bf16(FwdArgs a, bool vec_n, hipStream_t stream) {
  constexpr int BM = 32 * kWaves;
  a.q_tiles = (a.n_q + BM - 1) / BM;
  const dim3 grid(static_cast<unsigned>(a.BH) * a.q_tiles);
  if (vec_n)
    attn_fwd_bf16<KD, DV, kNCHW, true, kWaves><<<grid, kWaves * 64, 0, stream>>>(a);
  else
    attn_fwd_bf16<KD, DV, kNCHW, false, kWaves><<<grid, kWaves * 64, 0, stream>>>(a);
  return hipGetLastError();
}

template <int KD, bool kNCHW>
hipError_t run_f32(FwdArgsF32 a, hipStream_t stream) {
  const unsigned q_blocks = (a.n_q + kF32Threads - 1) / kF32Threads;
  const dim3 grid(q_blocks * a.BH * (kNCHW ? 2 : 1));
  attn_fwd_f32<KD, kNCHW><<<grid, kF32Threads, 0, stream>>>(a);
  return hipGetLastError();
}

constexpr int kWavesFwd = 4;

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
