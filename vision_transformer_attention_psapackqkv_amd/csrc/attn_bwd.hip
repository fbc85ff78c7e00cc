// Flash Attention 2 backward for gfx950.
//
// vision-rs book, "Custom Kernels", section "Flash Attention 2": the dQ
// backward and the dK/dV backward are separate kernels, each with its own
// grid. With P = exp(scale*Q K^T - LSE) recomputed from the forward's LSE,
// Delta = rowsum(dO * O) and dS = P * (dO V^T - Delta):
//   dV = P^T dO,   dK = scale * dS^T Q,   dQ = scale * dS K.
// Head dims 32..128 take two launches: dQ (one workgroup per query tile,
// looping over key tiles), which also computes Delta for its query rows from
// the O and dO rows it loads and stores it negated (the dP accumulators start
// from -Delta) beside LSE * log2(e), then dK/dV (one workgroup per key tile,
// looping over query tiles), which reads both. Head dim 16, batch-heads of
// 2 GB or more and the float32 path run a separate Delta pass first. No kernel
// uses atomics.
//
// The matrix-core products use v_mfma_f32_32x32x16_bf16 with the operand
// placement of the forward kernel: the rows of the first products' LDS
// operands are permuted (key_of_row) so that their accumulators (the scores,
// P and dS) are already the register operands of the next products, and the
// LDS operands of those products, whose reduction index runs down the staged
// rows, are read from the same row tiles with transposed LDS reads
// (ds_read_b64_tr_b16). Head dims 32..128 stage their tiles straight from
// global memory into swizzled unpadded rows; head dim 16 through registers
// into padded rows. The float32 path runs on the VALU, four lanes per row.
#include <math.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>

#include "psa_device.hpp"
#include "psa_launch.hpp"

namespace psa {
namespace {

constexpr int kPad = 8;

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;     // natural log, [BH, n_q]
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* delta;         // -Delta = -rowsum(dO o), [BH, n_q]
  float* lse2;          // LSE * log2(e), [BH, n_q]
  int BH, n_q, n_k;
  int tiles;            // workgroups per batch-head
  float scale;
  float c;              // scale * log2(e)
  int bh0;              // float32 kernels: first batch-head of this launch
};


__device__ __forceinline__ void block_of(int total, int tiles, int& bh, int& t) {
  const int i = blockIdx.x;
  const int per = total / 8;
  const int L = (i < per * 8) ? (i % 8) * per + i / 8 : i;   // XCD-contiguous runs
  bh = L / tiles;
  t = L - bh * tiles;
}

// ---------------------------------------------------------------- Delta

template <int D, bool kBf16>
__global__ __launch_bounds__(256) void bwd_delta(BwdArgs a) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (row >= static_cast<int64_t>(a.BH) * a.n_q) return;
  float acc = 0.0f;
  if constexpr (kBf16) {
    const uint16_t* o = a.o + row * D;
    const uint16_t* g = a.dout + row * D;
#pragma unroll
    for (int c = 0; c < D / 8; ++c) {
      const u32x4 ov = load16(o + c * 8), gv = load16(g + c * 8);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        acc = fmaf(__builtin_bit_cast(float, ov[w] << 16), __builtin_bit_cast(float, gv[w] << 16), acc);
        acc = fmaf(__builtin_bit_cast(float, ov[w] & 0xFFFF0000u),
                   __builtin_bit_cast(float, gv[w] & 0xFFFF0000u), acc);
      }
    }
  } else {
    const float* o = reinterpret_cast<const float*>(a.o) + row * D;
    const float* g = reinterpret_cast<const float*>(a.dout) + row * D;
#pragma unroll
    for (int d = 0; d < D; ++d) acc = fmaf(o[d], g[d], acc);
  }
  a.delta[row] = -acc;   // stored negated: the dP accumulators start from it
  a.lse2[row] = a.lse[row] * kLog2e;
}

// ---------------------------------------------------------------- dK / dV (bf16)

template <int D, int kWaves>
struct DkdvTile {
  static constexpr int NT = kWaves * 64;
  static constexpr int BQ = 64;                    // queries per tile
  static constexpr int DP = D < 32 ? 32 : D;       // dK/dV rows in whole 32-row blocks
  static constexpr int RSTR = D + kPad;            // [q][d] tiles
  static constexpr int R_ELEMS = BQ * RSTR;
  // Layout of one buffer (bf16 elements, then floats).
  static constexpr int OFF_Q = 0, OFF_DO = R_ELEMS;
  static constexpr int H_ELEMS = 2 * R_ELEMS;      // bf16 elements (even count)
  static constexpr int BUF_BYTES = H_ELEMS * 2 + 2 * BQ * 4;
  static constexpr int CHUNKS = BQ * D / 8;        // 16-byte pieces of the Q (and of the dO) rows
  static constexpr int PER = (CHUNKS + NT - 1) / NT;

  // Raw loads of the next tile. Every load is unconditional (chunk and row
  // indices clamped into range) and nothing reads the loaded registers until
  // store() at the end of the current tile, so the loads stay in flight while
  // it is computed; store() zeroes the rows past n_q.
  u32x4 qr[PER], gr[PER];
  float l2, dl;
  int rows;   // rows of this tile that exist (n_q - first row)

  __device__ __forceinline__ void load(const BwdArgs& a, int bh, int qt, int tid) {
    const int q0 = qt * BQ;
    rows = a.n_q - q0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = tid + i * NT;
      const int cc = c < CHUNKS ? c : CHUNKS - 1;
      const int r = cc / (D / 8), cb = cc % (D / 8);
      const int64_t off = (static_cast<int64_t>(bh) * a.n_q + min(q0 + r, a.n_q - 1)) * D + cb * 8;
      qr[i] = load16(a.q + off);
      gr[i] = load16(a.dout + off);
    }
    const int64_t i = static_cast<int64_t>(bh) * a.n_q + min(q0 + (tid < BQ ? tid : BQ - 1), a.n_q - 1);
    l2 = a.lse[i];
    dl = a.delta[i];
  }

  __device__ __forceinline__ void store(char* buf, int tid) const {
    uint16_t* h = reinterpret_cast<uint16_t*>(buf);
    float* f = reinterpret_cast<float*>(buf + H_ELEMS * 2);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = tid + i * NT;
      if (c < CHUNKS) {
        const int r = c / (D / 8), cb = c % (D / 8);
        const bool ok = r < rows;
        *reinterpret_cast<u32x4*>(h + OFF_Q + r * RSTR + cb * 8) = ok ? qr[i] : zero4();
        *reinterpret_cast<u32x4*>(h + OFF_DO + r * RSTR + cb * 8) = ok ? gr[i] : zero4();
      }
    }
    if (tid < BQ) {
      // Rows past n_q get P = 0 (LSE = +inf) and Delta = 0.
      const bool ok = tid < rows;
      f[tid] = ok ? l2 * kLog2e : INFINITY;
      f[BQ + tid] = ok ? dl : 0.0f;
    }
  }
};

// Registers capped for three workgroups per CU up to head dim 32 and for two
// at 64 (both fit without spilling; measured faster than fewer workgroups with
// more registers); head dim 128 needs a whole SIMD's register file.
template <int D, int kWaves>
__global__ __launch_bounds__(kWaves * 64, D <= 32 ? 3 : D == 64 ? 2 : 1) void bwd_dkdv_bf16(BwdArgs a) {
  using Tile = DkdvTile<D, kWaves>;
  constexpr int BQ = Tile::BQ;
  constexpr int NDS = D / 16;
  constexpr int NDB = Tile::DP / 32;
  __shared__ __attribute__((aligned(16))) char smem[2 * Tile::BUF_BYTES];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, g = lane >> 5;
  const int i16 = lane & 15, t16 = (lane >> 4) & 1;
  int bh, kt;
  block_of(a.BH * a.tiles, a.tiles, bh, kt);
  const int key = kt * 32 * kWaves + wave * 32 + l32;
  const bool k_ok = key < a.n_k;

  // This lane's key and value rows as B operands: K[key][16ds + 8g + j].
  // Keys past n_k load row n_k - 1 (all loads unconditional, in flight
  // together) and are zeroed afterwards.
  bf16x8 kop[NDS], vop[NDS];
  {
    u32x4 kr[NDS], vr[NDS];
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      const int64_t off = (static_cast<int64_t>(bh) * a.n_k + min(key, a.n_k - 1)) * D + ds * 16 + g * 8;
      kr[ds] = load16(a.k + off);
      vr[ds] = load16(a.v + off);
    }
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      kop[ds] = as_bf16x8(k_ok ? kr[ds] : zero4());
      vop[ds] = as_bf16x8(k_ok ? vr[ds] : zero4());
    }
  }
  f32x16 dk_acc[NDB], dv_acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dk_acc[db][r] = dv_acc[db][r] = 0.0f;

  const int n_tiles = (a.n_q + BQ - 1) / BQ;
  Tile tile;
  tile.load(a, bh, 0, tid);
  tile.store(smem, tid);
  __syncthreads();

  for (int qt = 0; qt < n_tiles; ++qt) {
    const char* buf = smem + (qt & 1) * Tile::BUF_BYTES;
    const uint16_t* h = reinterpret_cast<const uint16_t*>(buf);
    const float* f = reinterpret_cast<const float*>(buf + Tile::H_ELEMS * 2);
    const bool more = qt + 1 < n_tiles;
    if (more) tile.load(a, bh, qt + 1, tid);

#pragma unroll
    for (int qb = 0; qb < BQ / 32; ++qb) {
      // S[q][key] = Q K^T and dP[q][key] = dO V^T for 32 queries. Row rho of the
      // A operands is query key_of_row(rho), so element r of lane group g holds
      // query qb*32 + 16*(r/8) + 8g + r%8 (P and dS come out as B operands over
      // 8 consecutive queries); dP's accumulator starts at -Delta, so it ends as
      // dP - Delta.
      f32x16 sacc, pacc;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 dl = *reinterpret_cast<const f32x4*>(f + BQ + qb * 32 + 16 * (r4 >> 1) + 8 * g + 4 * (r4 & 1));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sacc[4 * r4 + e] = 0.0f;
          pacc[4 * r4 + e] = dl[e];   // -Delta
        }
      }
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        const int off = (qb * 32 + key_of_row(l32)) * Tile::RSTR + ds * 16 + g * 8;
        sacc = mfma32x32x16(*reinterpret_cast<const bf16x8*>(h + Tile::OFF_Q + off), kop[ds], sacc);
        pacc = mfma32x32x16(*reinterpret_cast<const bf16x8*>(h + Tile::OFF_DO + off), vop[ds], pacc);
      }
      // P and dS.
      bf16x8 pb[2], sb[2];
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 l2 = *reinterpret_cast<const f32x4*>(f + qb * 32 + 16 * (r4 >> 1) + 8 * g + 4 * (r4 & 1));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * r4 + e;
          const float p = fast_exp2(fmaf(sacc[r], a.c, -l2[e]));
          pb[r >> 3][r & 7] = static_cast<__bf16>(p);
          sb[r >> 3][r & 7] = static_cast<__bf16>(p * pacc[r]);
        }
      }
      // dV^T += dO^T P,  dK^T += Q^T dS  (reduction over the 32 queries, 2 steps of
      // 16). dO^T and Q^T come from the row tiles through transposed LDS reads; with
      // D = 16 the second 16-row half of the block reads past the row (finite data)
      // and is zeroed: those rows are never stored.
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int off = ((qb * 2 + s) * 16 + 8 * g + (i16 >> 2)) * Tile::RSTR + db * 32 + 16 * t16 + 4 * (i16 & 3);
          bf16x8 gt = lds_read_tr8(h + Tile::OFF_DO + off, Tile::RSTR);
          bf16x8 qt_op = lds_read_tr8(h + Tile::OFF_Q + off, Tile::RSTR);
          if constexpr (Tile::DP > D) {
            if (db * 32 + l32 >= D) gt = qt_op = as_bf16x8(zero4());
          }
          dv_acc[db] = mfma32x32x16(gt, pb[s], dv_acc[db]);
          dk_acc[db] = mfma32x32x16(qt_op, sb[s], dk_acc[db]);
        }
    }
    if (more) tile.store(smem + ((qt + 1) & 1) * Tile::BUF_BYTES, tid);
    __syncthreads();
  }

  if (!k_ok) return;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d0 = db * 32 + 8 * r4 + 4 * g;
      if (d0 >= D) continue;
      const int64_t off = (static_cast<int64_t>(bh) * a.n_k + key) * D + d0;
      uint32_t kw[2], vw[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        kw[e] = float_to_bf16_bits(dk_acc[db][4 * r4 + 2 * e] * a.scale) |
                (uint32_t(float_to_bf16_bits(dk_acc[db][4 * r4 + 2 * e + 1] * a.scale)) << 16);
        vw[e] = float_to_bf16_bits(dv_acc[db][4 * r4 + 2 * e]) |
                (uint32_t(float_to_bf16_bits(dv_acc[db][4 * r4 + 2 * e + 1])) << 16);
      }
      *reinterpret_cast<u32x2*>(a.dk + off) = u32x2{kw[0], kw[1]};
      *reinterpret_cast<u32x2*>(a.dv + off) = u32x2{vw[0], vw[1]};
    }
}

// ---------------------------------------------------------------- dQ (bf16)

template <int D, int kWaves>
struct DqTile {
  static constexpr int NT = kWaves * 64;
  static constexpr int BN = 64;                    // keys per tile
  static constexpr int DP = D < 32 ? 32 : D;       // dQ rows in whole 32-row blocks
  static constexpr int RSTR = D + kPad;
  static constexpr int R_ELEMS = BN * RSTR;
  static constexpr int OFF_K = 0, OFF_V = R_ELEMS;
  static constexpr int BUF = 2 * R_ELEMS;
  static constexpr int CHUNKS = BN * D / 8;        // 16-byte pieces of the K (and of the V) rows
  static constexpr int PER = (CHUNKS + NT - 1) / NT;

  // Raw loads of the next tile: unconditional (indices clamped into range),
  // not read until store() at the end of the current tile, which zeroes the
  // rows past n_k.
  u32x4 kr[PER];
  u32x4 vr[PER];
  int rows;   // rows of this tile that exist (n_k - first row)

  __device__ __forceinline__ void load(const BwdArgs& a, int bh, int kt, int tid) {
    const int m0 = kt * BN;
    rows = a.n_k - m0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = tid + i * NT;
      const int cc = c < CHUNKS ? c : CHUNKS - 1;
      const int r = cc / (D / 8), cb = cc % (D / 8);
      const int64_t off = (static_cast<int64_t>(bh) * a.n_k + min(m0 + r, a.n_k - 1)) * D + cb * 8;
      kr[i] = load16(a.k + off);
      vr[i] = load16(a.v + off);
    }
  }

  __device__ __forceinline__ void store(uint16_t* buf, int tid) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = tid + i * NT;
      if (c < CHUNKS) {
        const int r = c / (D / 8), cb = c % (D / 8);
        const bool ok = r < rows;
        *reinterpret_cast<u32x4*>(buf + OFF_K + r * RSTR + cb * 8) = ok ? kr[i] : zero4();
        *reinterpret_cast<u32x4*>(buf + OFF_V + r * RSTR + cb * 8) = ok ? vr[i] : zero4();
      }
    }
  }
};

template <int D, int kWaves>
__global__ __launch_bounds__(kWaves * 64, D <= 32 ? 3 : D == 64 ? 2 : 1) void bwd_dq_bf16(BwdArgs a) {
  using Tile = DqTile<D, kWaves>;
  constexpr int BN = Tile::BN;
  constexpr int NDS = D / 16;
  constexpr int NDB = Tile::DP / 32;
  constexpr int BM = 32 * kWaves;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * Tile::BUF];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l32 = lane & 31, g = lane >> 5;
  const int i16 = lane & 15, t16 = (lane >> 4) & 1;
  int bh, qt;
  block_of(a.BH * a.tiles, a.tiles, bh, qt);
  const int q = qt * BM + wave * 32 + l32;
  const bool q_ok = q < a.n_q;

  // Queries past n_q load row n_q - 1 (all loads unconditional, in flight
  // together) and are zeroed afterwards.
  bf16x8 qop[NDS], gop[NDS];
  float l2, dl;
  {
    const int qc = min(q, a.n_q - 1);
    u32x4 qr[NDS], gr[NDS];
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      const int64_t off = (static_cast<int64_t>(bh) * a.n_q + qc) * D + ds * 16 + g * 8;
      qr[ds] = load16(a.q + off);
      gr[ds] = load16(a.dout + off);
    }
    const float lv = a.lse[static_cast<int64_t>(bh) * a.n_q + qc];
    const float dv = a.delta[static_cast<int64_t>(bh) * a.n_q + qc];
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      qop[ds] = as_bf16x8(q_ok ? qr[ds] : zero4());
      gop[ds] = as_bf16x8(q_ok ? gr[ds] : zero4());
    }
    l2 = q_ok ? lv * kLog2e : 0.0f;
    dl = q_ok ? dv : 0.0f;
  }
  f32x16 dq_acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq_acc[db][r] = 0.0f;

  const int n_tiles = (a.n_k + BN - 1) / BN;
  Tile tile;
  tile.load(a, bh, 0, tid);
  tile.store(smem, tid);
  __syncthreads();

  // One key tile. Only the last tile (`last` true) can hold keys past n_k,
  // and only its code masks them: a run-time test on every tile is flattened
  // by the compiler into a compare and a select per score.
  auto step = [&](int kt, auto last) __attribute__((always_inline)) {
    const uint16_t* buf = smem + (kt & 1) * Tile::BUF;
    const bool more = kt + 1 < n_tiles;
    if (more) tile.load(a, bh, kt + 1, tid);

    bf16x8 sb[BN / 16];
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
      // S^T[key][q] = K Q^T and dP^T[key][q] = V dO^T (its accumulator starts at
      // -Delta, so it ends as dP^T - Delta). Row rho of the A operands is key
      // key_of_row(rho), so element r of lane group g holds key 16*(r/8) + 8g + r%8
      // of the block: the dS values come out as B operands of the dQ product.
      f32x16 sacc, pacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sacc[r] = 0.0f;
        pacc[r] = dl;   // -Delta
      }
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        const int off = (kb * 32 + key_of_row(l32)) * Tile::RSTR + ds * 16 + g * 8;
        sacc = mfma32x32x16(*reinterpret_cast<const bf16x8*>(buf + Tile::OFF_K + off), qop[ds], sacc);
        pacc = mfma32x32x16(*reinterpret_cast<const bf16x8*>(buf + Tile::OFF_V + off), gop[ds], pacc);
      }
      // Keys past n_k get P = 0.
      if constexpr (decltype(last)::value) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kt * BN + kb * 32 + 16 * (r >> 3) + 8 * g + (r & 7) >= a.n_k) sacc[r] = -INFINITY;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(fmaf(sacc[r], a.c, -l2));
        sb[kb * 2 + (r >> 3)][r & 7] = static_cast<__bf16>(p * pacc[r]);
      }
    }
    // dQ^T += K^T dS^T (reduction over the tile's keys); K^T comes from the K rows
    // through transposed LDS reads. With D = 16 the second 16-row half of the
    // block reads past the row (finite data) and is zeroed: those dQ rows are
    // never stored.
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int s = 0; s < BN / 16; ++s) {
        bf16x8 kop = lds_read_tr8(buf + Tile::OFF_K + (s * 16 + 8 * g + (i16 >> 2)) * Tile::RSTR + db * 32 +
                                      16 * t16 + 4 * (i16 & 3),
                                  Tile::RSTR);
        if constexpr (Tile::DP > D) {
          if (db * 32 + l32 >= D) kop = as_bf16x8(zero4());
        }
        dq_acc[db] = mfma32x32x16(kop, sb[s], dq_acc[db]);
      }
    if (more) tile.store(smem + ((kt + 1) & 1) * Tile::BUF, tid);
    __syncthreads();
  };
  for (int kt = 0; kt + 1 < n_tiles; ++kt) step(kt, std::false_type{});
  step(n_tiles - 1, std::true_type{});

  if (!q_ok) return;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d0 = db * 32 + 8 * r4 + 4 * g;
      if (d0 >= D) continue;
      uint32_t w[2];
#pragma unroll
      for (int e = 0; e < 2; ++e)
        w[e] = float_to_bf16_bits(dq_acc[db][4 * r4 + 2 * e] * a.scale) |
               (uint32_t(float_to_bf16_bits(dq_acc[db][4 * r4 + 2 * e + 1] * a.scale)) << 16);
      *reinterpret_cast<u32x2*>(a.dq + (static_cast<int64_t>(bh) * a.n_q + q) * D + d0) = u32x2{w[0], w[1]};
    }
}

// ---------------------------------------------------------------- direct staging (D >= 32)
//
// Head dims 32..128 with rows under 2 GB per batch-head stage their tiles
// straight from global memory into LDS (buffer loads with an LDS destination):
// no registers hold tile data and no LDS write or address instruction is
// spent per tile. Tiles are 64 unpadded rows whose 16-byte chunks are placed
// by packed_chunk_pos<D>, which keeps both read patterns of these kernels (the
// 16-byte A-operand reads in key_of_row order and the transposed reads of rows
// r and r + 4) free of bank conflicts. Rows past n lie outside the buffer
// and read as zero: a zero Q/dO row (dK/dV kernel) or K/V row (dQ kernel)
// contributes nothing to any product, so no tile is masked.

// One 64-row tile of a [n][D] tensor: wave instruction b fills 1 KB block b
// (512 / D rows), lane i the i-th chunk, fetching the global chunk the swizzle
// puts there. The lane's offset is the same for every tile; the tile's first
// row is a scalar offset. kUser tells the two kernels' instances apart: with
// one instance shared by both kernels, this compiler left the host stub of the
// second kernel launched undefined.
template <int D, int kWaves, int kUser>
struct RowStage {
  static constexpr int CPR = D / 8;                    // chunks per row
  static constexpr int RPB = 64 / CPR;                 // rows per 1 KB block
  static constexpr int BLOCKS = 64 / RPB;
  static constexpr int PER = (BLOCKS + kWaves - 1) / kWaves;
  uint32_t voff[PER];

  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int row = (wave + i * kWaves) * RPB + lane / CPR;
      voff[i] = static_cast<uint32_t>(row * D + packed_chunk_pos<D>(row, lane % CPR) * 8) * 2u;   // an involution
    }
  }

  // `wave` must be wave-uniform.
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rsrc, int row0, uint16_t* tile, int wave) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int b = wave + i * kWaves;
      if (BLOCKS % kWaves != 0 && b >= BLOCKS) break;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)(tile + b * 512),
                                               16, voff[i], row0 * D * 2, 0, 0);
    }
  }
};

// 16 bytes of row `row`, chunk c, of a swizzled [64][D] tile.
template <int D>
__device__ __forceinline__ bf16x8 row_read8(const uint16_t* t, int row, int c) {
  return *reinterpret_cast<const bf16x8*>(t + row * D + packed_chunk_pos<D>(row, c) * 8);
}

// One operand of 8 values down rows r .. r+7 at column col of a swizzled
// [64][D] tile: transposed reads of rows r.. and r+4.. (see lds_read_tr8).
template <int D>
__device__ __forceinline__ bf16x8 row_read_tr8(const uint16_t* t, int r, int col) {
  return lds_read_tr8_2(t + r * D + packed_chunk_pos<D>(r, col >> 3) * 8 + (col & 7),
                        t + (r + 4) * D + packed_chunk_pos<D>(r + 4, col >> 3) * 8 + (col & 7));
}

template <int D, int kWaves>
__global__ __launch_bounds__(kWaves * 64, D <= 32 ? 3 : D == 64 ? 2 : 1) void bwd_dkdv_direct(BwdArgs a) {
  constexpr int BQ = 64;                 // queries per tile
  constexpr int NDS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int T_EL = BQ * D;           // bf16 elements of one row tile
  constexpr int BUF = 2 * T_EL + 4 * BQ; // Q and dO tiles, then LSE*log2(e) and -Delta (floats)
  // Two tile buffers as two objects reached through restrict pointers, so the
  // LDS reads of one tile need not wait for the direct loads into the other.
  __shared__ __attribute__((aligned(16))) uint16_t smem0[BUF];
  __shared__ __attribute__((aligned(16))) uint16_t smem1[BUF];

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i16 = lane & 15, t16 = (lane >> 4) & 1;
  int bh, kt;
  block_of(a.BH * a.tiles, a.tiles, bh, kt);
  const int key = kt * 32 * kWaves + wave * 32 + l32;
  const bool k_ok = key < a.n_k;

  // Tile sources: this batch-head's Q and dO rows and its LSE*log2(e) and
  // -Delta values (each buffer ends at row n_q: rows past it read as zero).
  const int64_t rows0 = static_cast<int64_t>(bh) * a.n_q;
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.q + rows0 * D), 0, a.n_q * D * 2, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rg = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.dout + rows0 * D), 0, a.n_q * D * 2, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(a.lse2 + rows0, 0, a.n_q * 4, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(a.delta + rows0, 0, a.n_q * 4, kBufferWord3);
  RowStage<D, kWaves, 0> st;
  st.init(wave, lane);
  auto issue = [&](int qt, uint16_t* buf) {
    st.issue(rq, qt * BQ, buf, wave);
    st.issue(rg, qt * BQ, buf + T_EL, wave);
    float* f = reinterpret_cast<float*>(buf + 2 * T_EL);
    if (wave == 0)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (__attribute__((address_space(3))) void*)f, 4, lane * 4u,
                                               qt * BQ * 4, 0, 0);
    else if (wave == 1)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (__attribute__((address_space(3))) void*)(f + BQ), 4,
                                               lane * 4u, qt * BQ * 4, 0, 0);
  };
  const int n_tiles = (a.n_q + BQ - 1) / BQ;
  issue(0, smem0);

  // This lane's key and value rows as B operands: K[key][16ds + 8g + j]. Keys
  // past n_k load row n_k - 1 (every load unconditional, all in flight
  // together) and are zeroed afterwards.
  bf16x8 kop[NDS], vop[NDS];
  {
    u32x4 kr[NDS], vr[NDS];
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      const int64_t off = (static_cast<int64_t>(bh) * a.n_k + min(key, a.n_k - 1)) * D + ds * 16 + g * 8;
      kr[ds] = load16(a.k + off);
      vr[ds] = load16(a.v + off);
    }
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      kop[ds] = as_bf16x8(k_ok ? kr[ds] : zero4());
      vop[ds] = as_bf16x8(k_ok ? vr[ds] : zero4());
    }
  }
  f32x16 dk_acc[NDB], dv_acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dk_acc[db][r] = dv_acc[db][r] = 0.0f;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's part of tile 0 landed
  __syncthreads();

  // One query tile, read from h while the next one is loaded into nbuf.
  auto tile = [&](int qt, const uint16_t* __restrict__ h, uint16_t* __restrict__ nbuf)
                  __attribute__((always_inline)) {
    const uint16_t* hg = h + T_EL;
    const float* f = reinterpret_cast<const float*>(h + 2 * T_EL);
    if (qt + 1 < n_tiles) issue(qt + 1, nbuf);

    // The two 32-query blocks unrolled (every LDS address a per-lane offset
    // plus a constant: the swizzle does not depend on the block) and kept one
    // after the other by a scheduling barrier, so their registers do not overlap.
#pragma unroll
    for (int qb = 0; qb < BQ / 32; ++qb) {
      if (qb > 0) __builtin_amdgcn_sched_barrier(0);
      // S[q][key] = Q K^T and dP[q][key] = dO V^T for 32 queries. Row rho of the
      // A operands is query key_of_row(rho), so element r of lane group g holds
      // query qb*32 + 16*(r/8) + 8g + r%8; dP's accumulator starts at -Delta.
      f32x16 sacc, pacc;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 dl = *reinterpret_cast<const f32x4*>(f + BQ + qb * 32 + 16 * (r4 >> 1) + 8 * g + 4 * (r4 & 1));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sacc[4 * r4 + e] = 0.0f;
          pacc[4 * r4 + e] = dl[e];
        }
      }
      const int row = qb * 32 + key_of_row(l32);
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        sacc = mfma32x32x16(row_read8<D>(h, row, ds * 2 + g), kop[ds], sacc);
        pacc = mfma32x32x16(row_read8<D>(hg, row, ds * 2 + g), vop[ds], pacc);
      }
      bf16x8 pb[2], sb[2];
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 l2 = *reinterpret_cast<const f32x4*>(f + qb * 32 + 16 * (r4 >> 1) + 8 * g + 4 * (r4 & 1));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * r4 + e;
          const float p = fast_exp2(fmaf(sacc[r], a.c, -l2[e]));
          pb[r >> 3][r & 7] = static_cast<__bf16>(p);
          sb[r >> 3][r & 7] = static_cast<__bf16>(p * pacc[r]);
        }
      }
      // dV^T += dO^T P,  dK^T += Q^T dS over the block's queries, 16 per step.
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int r = (qb * 2 + s) * 16 + 8 * g + (i16 >> 2);
          const int col = db * 32 + 16 * t16 + 4 * (i16 & 3);
          dv_acc[db] = mfma32x32x16(row_read_tr8<D>(hg, r, col), pb[s], dv_acc[db]);
          dk_acc[db] = mfma32x32x16(row_read_tr8<D>(h, r, col), sb[s], dk_acc[db]);
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's part of the next tile landed
    __syncthreads();
  };
  // A wave whose 32 keys all lie past n_k (the last key tile of a batch-head
  // when n_k is not a multiple of 128) only helps stage the tiles and meets
  // the barriers, in a loop of its own (a branch inside the loop below would
  // cost it registers).
  if (kt * 32 * kWaves + wave * 32 >= a.n_k) {
    for (int t = 0; t < n_tiles; ++t) {
      if (t + 1 < n_tiles) issue(t + 1, (t & 1) ? smem0 : smem1);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }
    return;
  }
  // Tile t lives in smem0 for even t, smem1 for odd. Two tiles per trip, so
  // that each one reads a fixed LDS object: every LDS address is then a
  // loop-invariant per-lane offset plus a constant.
  int qt = 0;
  for (; qt + 1 < n_tiles; qt += 2) {
    tile(qt, smem0, smem1);
    tile(qt + 1, smem1, smem0);
  }
  if (qt < n_tiles) tile(qt, smem0, smem1);

  if (!k_ok) return;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d0 = db * 32 + 8 * r4 + 4 * g;
      const int64_t off = (static_cast<int64_t>(bh) * a.n_k + key) * D + d0;
      uint32_t kw[2], vw[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        kw[e] = float_to_bf16_bits(dk_acc[db][4 * r4 + 2 * e] * a.scale) |
                (uint32_t(float_to_bf16_bits(dk_acc[db][4 * r4 + 2 * e + 1] * a.scale)) << 16);
        vw[e] = float_to_bf16_bits(dv_acc[db][4 * r4 + 2 * e]) |
                (uint32_t(float_to_bf16_bits(dv_acc[db][4 * r4 + 2 * e + 1])) << 16);
      }
      *reinterpret_cast<u32x2*>(a.dk + off) = u32x2{kw[0], kw[1]};
      *reinterpret_cast<u32x2*>(a.dv + off) = u32x2{vw[0], vw[1]};
    }
}

// Registers capped for four workgroups per CU at head dim 32 (128 VGPRs, no
// spills; left free, the compiler takes 131 and the kernel runs three).
template <int D, int kWaves>
__global__ __launch_bounds__(kWaves * 64, D <= 32 ? 4 : D == 64 ? 2 : 1) void bwd_dq_direct(BwdArgs a) {
  constexpr int BN = 64;                 // keys per tile
  constexpr int NDS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int BM = 32 * kWaves;
  constexpr int T_EL = BN * D;
  __shared__ __attribute__((aligned(16))) uint16_t smem0[2 * T_EL];
  __shared__ __attribute__((aligned(16))) uint16_t smem1[2 * T_EL];

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i16 = lane & 15, t16 = (lane >> 4) & 1;
  int bh, qt;
  block_of(a.BH * a.tiles, a.tiles, bh, qt);
  const int q = qt * BM + wave * 32 + l32;
  const bool q_ok = q < a.n_q;

  const int64_t keys0 = static_cast<int64_t>(bh) * a.n_k;
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.k + keys0 * D), 0, a.n_k * D * 2, kBufferWord3);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.v + keys0 * D), 0, a.n_k * D * 2, kBufferWord3);
  RowStage<D, kWaves, 1> st;
  st.init(wave, lane);
  auto issue = [&](int kt, uint16_t* buf) {
    st.issue(rk, kt * BN, buf, wave);
    st.issue(rv, kt * BN, buf + T_EL, wave);
  };
  const int n_tiles = (a.n_k + BN - 1) / BN;
  issue(0, smem0);

  // This lane's query and dO rows as B operands. Queries past n_q load row
  // n_q - 1 (all loads unconditional) and are zeroed afterwards; they are
  // never stored. This kernel runs first and also computes, for its queries,
  // -Delta = -rowsum(dO o O) (lanes l and l ^ 32 each hold half of a row) and
  // LSE * log2(e), and stores both for the dK/dV kernel.
  bf16x8 qop[NDS], gop[NDS];
  float l2, dl;
  {
    const int qc = min(q, a.n_q - 1);
    const int64_t row = static_cast<int64_t>(bh) * a.n_q + qc;
    u32x4 qr[NDS], gr[NDS], orow[NDS];
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      const int64_t off = row * D + ds * 16 + g * 8;
      qr[ds] = load16(a.q + off);
      gr[ds] = load16(a.dout + off);
      orow[ds] = load16(a.o + off);
    }
    const float lv = a.lse[row] * kLog2e;
    float part = 0.0f;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        part = fmaf(__builtin_bit_cast(float, orow[ds][w] << 16), __builtin_bit_cast(float, gr[ds][w] << 16), part);
        part = fmaf(__builtin_bit_cast(float, orow[ds][w] & 0xFFFF0000u),
                    __builtin_bit_cast(float, gr[ds][w] & 0xFFFF0000u), part);
      }
    const float dv = -(part + __shfl_xor(part, 32));
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      qop[ds] = as_bf16x8(q_ok ? qr[ds] : zero4());
      gop[ds] = as_bf16x8(q_ok ? gr[ds] : zero4());
    }
    l2 = q_ok ? lv : 0.0f;
    dl = q_ok ? dv : 0.0f;
    if (q_ok && g == 0) {
      a.delta[row] = dv;
      a.lse2[row] = lv;
    }
  }
  f32x16 dq_acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq_acc[db][r] = 0.0f;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's part of tile 0 landed
  __syncthreads();

  auto tile = [&](int kt, const uint16_t* __restrict__ ks, uint16_t* __restrict__ nbuf)
                  __attribute__((always_inline)) {
    const uint16_t* vs = ks + T_EL;
    if (kt + 1 < n_tiles) issue(kt + 1, nbuf);
    bf16x8 sb[BN / 16];
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
      // S^T[key][q] = K Q^T and dP^T[key][q] = V dO^T (from -Delta). Row rho of
      // the A operands is key key_of_row(rho): element r of lane group g holds
      // key 16*(r/8) + 8g + r%8 of the block, so dS comes out as the B operand
      // of the dQ product.
      f32x16 sacc, pacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sacc[r] = 0.0f;
        pacc[r] = dl;
      }
      const int row = kb * 32 + key_of_row(l32);
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
        sacc = mfma32x32x16(row_read8<D>(ks, row, ds * 2 + g), qop[ds], sacc);
        pacc = mfma32x32x16(row_read8<D>(vs, row, ds * 2 + g), gop[ds], pacc);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(fmaf(sacc[r], a.c, -l2));
        sb[kb * 2 + (r >> 3)][r & 7] = static_cast<__bf16>(p * pacc[r]);
      }
    }
    // dQ^T += K^T dS^T over the tile's keys; K^T through transposed reads.
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int s = 0; s < BN / 16; ++s)
        dq_acc[db] = mfma32x32x16(row_read_tr8<D>(ks, s * 16 + 8 * g + (i16 >> 2), db * 32 + 16 * t16 + 4 * (i16 & 3)),
                                  sb[s], dq_acc[db]);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's part of the next tile landed
    __syncthreads();
  };
  // A wave whose 32 queries all lie past n_q only helps stage the tiles, as in
  // the dK/dV kernel.
  if (qt * BM + wave * 32 >= a.n_q) {
    for (int t = 0; t < n_tiles; ++t) {
      if (t + 1 < n_tiles) issue(t + 1, (t & 1) ? smem0 : smem1);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }
    return;
  }
  int kt = 0;   // two tiles per trip, as in the dK/dV kernel
  for (; kt + 1 < n_tiles; kt += 2) {
    tile(kt, smem0, smem1);
    tile(kt + 1, smem1, smem0);
  }
  if (kt < n_tiles) tile(kt, smem0, smem1);

  if (!q_ok) return;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d0 = db * 32 + 8 * r4 + 4 * g;
      uint32_t w[2];
#pragma unroll
      for (int e = 0; e < 2; ++e)
        w[e] = float_to_bf16_bits(dq_acc[db][4 * r4 + 2 * e] * a.scale) |
               (uint32_t(float_to_bf16_bits(dq_acc[db][4 * r4 + 2 * e + 1] * a.scale)) << 16);
      *reinterpret_cast<u32x2*>(a.dq + (static_cast<int64_t>(bh) * a.n_q + q) * D + d0) = u32x2{w[0], w[1]};
    }
}

// ---------------------------------------------------------------- float32

constexpr int kF32Threads = 128;
constexpr int kF32Rows = 32;                        // rows per LDS tile
constexpr int kF32Lanes = 4;                        // lanes per output row
constexpr int kF32Out = kF32Threads / kF32Lanes;    // output rows per workgroup

// Adds the partial sums x[0..D) of the four lanes of an output row (lanes
// 4i..4i+3); every lane ends with the total.
template <int D>
__device__ __forceinline__ void sum_lanes(float (&x)[D]) {
#pragma unroll
  for (int m = 1; m < kF32Lanes; m <<= 1)
#pragma unroll
    for (int d = 0; d < D; ++d) x[d] += __shfl_xor(x[d], m);
}

// dK/dV: four lanes per key, lane l taking queries l, l+4, ... of each tile
// (staged through LDS); the lanes' partial dK and dV are added at the end and
// each lane stores the columns d = l (mod 4).
template <int D>
__global__ __launch_bounds__(kF32Threads) void bwd_dkdv_f32(BwdArgs a) {
  __shared__ float qs[kF32Rows][D];
  __shared__ float gs[kF32Rows][D];
  __shared__ float ls[kF32Rows], dls[kF32Rows];
  const float* Q = reinterpret_cast<const float*>(a.q);
  const float* G = reinterpret_cast<const float*>(a.dout);
  const int blocks = (a.n_k + kF32Out - 1) / kF32Out;
  const int bh = a.bh0 + static_cast<int>(blockIdx.x / blocks);
  const int lane = threadIdx.x % kF32Lanes;
  const int key = (blockIdx.x % blocks) * kF32Out + threadIdx.x / kF32Lanes;
  const bool ok = key < a.n_k;
  float kr[D], vr[D], dk[D], dv[D];
  const int64_t krow = (static_cast<int64_t>(bh) * a.n_k + (ok ? key : 0)) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    kr[d] = ok ? reinterpret_cast<const float*>(a.k)[krow + d] : 0.0f;
    vr[d] = ok ? reinterpret_cast<const float*>(a.v)[krow + d] : 0.0f;
    dk[d] = dv[d] = 0.0f;
  }
  // Thread element i of a [kF32Rows, D] tile: row e / D, column e % D.
  auto rc = [](int i, int& r, int& d) {
    const int e = static_cast<int>(threadIdx.x) + i * kF32Threads;
    r = e / D;
    d = e % D;
  };
  for (int q0 = 0; q0 < a.n_q; q0 += kF32Rows) {
    __syncthreads();
    auto at = [&](int r, int d) { return (static_cast<int64_t>(bh) * a.n_q + q0 + r) * D + d; };
    move_batched<kF32Rows * D / kF32Threads>(
        [&](int i) { int r, d; rc(i, r, d); return q0 + r < a.n_q ? Q[at(r, d)] : 0.0f; },
        [&](int i, float x) { int r, d; rc(i, r, d); qs[r][d] = x; });
    move_batched<kF32Rows * D / kF32Threads>(
        [&](int i) { int r, d; rc(i, r, d); return q0 + r < a.n_q ? G[at(r, d)] : 0.0f; },
        [&](int i, float x) { int r, d; rc(i, r, d); gs[r][d] = x; });
    if (threadIdx.x < kF32Rows) {
      const int r = threadIdx.x;
      const bool in = q0 + r < a.n_q;
      ls[r] = in ? a.lse[static_cast<int64_t>(bh) * a.n_q + q0 + r] : 0.0f;
      dls[r] = in ? a.delta[static_cast<int64_t>(bh) * a.n_q + q0 + r] : 0.0f;
    }
    __syncthreads();
    const int cnt = min(kF32Rows, a.n_q - q0);
    for (int r = lane; r < cnt; r += kF32Lanes) {
      const float s = dot_f32<D>(qs[r], kr);
      const float dp = dot_f32<D>(gs[r], vr);
      const float p = expf(s * a.scale - ls[r]);
      const float ds = p * (dp + dls[r]);   // dls holds -Delta
#pragma unroll
      for (int d = 0; d < D; ++d) {
        dv[d] = fmaf(p, gs[r][d], dv[d]);
        dk[d] = fmaf(ds, qs[r][d], dk[d]);
      }
    }
  }
  sum_lanes<D>(dk);
  sum_lanes<D>(dv);
  if (!ok) return;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    if (d % kF32Lanes != lane) continue;
    reinterpret_cast<float*>(a.dk)[krow + d] = dk[d] * a.scale;
    reinterpret_cast<float*>(a.dv)[krow + d] = dv[d];
  }
}

// dQ: four lanes per query, lane l taking keys l, l+4, ... of each tile; the
// lanes' partial dQ are added at the end.
template <int D>
__global__ __launch_bounds__(kF32Threads) void bwd_dq_f32(BwdArgs a) {
  __shared__ float ks[kF32Rows][D];
  __shared__ float vs[kF32Rows][D];
  const float* K = reinterpret_cast<const float*>(a.k);
  const float* V = reinterpret_cast<const float*>(a.v);
  const int blocks = (a.n_q + kF32Out - 1) / kF32Out;
  const int bh = a.bh0 + static_cast<int>(blockIdx.x / blocks);
  const int lane = threadIdx.x % kF32Lanes;
  const int q = (blockIdx.x % blocks) * kF32Out + threadIdx.x / kF32Lanes;
  const bool ok = q < a.n_q;
  const int64_t qrow = (static_cast<int64_t>(bh) * a.n_q + (ok ? q : 0)) * D;
  float qr[D], gr[D], dq[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    qr[d] = ok ? reinterpret_cast<const float*>(a.q)[qrow + d] : 0.0f;
    gr[d] = ok ? reinterpret_cast<const float*>(a.dout)[qrow + d] : 0.0f;
    dq[d] = 0.0f;
  }
  const float lse = ok ? a.lse[static_cast<int64_t>(bh) * a.n_q + q] : 0.0f;
  const float dl = ok ? a.delta[static_cast<int64_t>(bh) * a.n_q + q] : 0.0f;
  auto rc = [](int i, int& r, int& d) {
    const int e = static_cast<int>(threadIdx.x) + i * kF32Threads;
    r = e / D;
    d = e % D;
  };
  for (int m0 = 0; m0 < a.n_k; m0 += kF32Rows) {
    __syncthreads();
    auto at = [&](int r, int d) { return (static_cast<int64_t>(bh) * a.n_k + m0 + r) * D + d; };
    move_batched<kF32Rows * D / kF32Threads>(
        [&](int i) { int r, d; rc(i, r, d); return m0 + r < a.n_k ? K[at(r, d)] : 0.0f; },
        [&](int i, float x) { int r, d; rc(i, r, d); ks[r][d] = x; });
    move_batched<kF32Rows * D / kF32Threads>(
        [&](int i) { int r, d; rc(i, r, d); return m0 + r < a.n_k ? V[at(r, d)] : 0.0f; },
        [&](int i, float x) { int r, d; rc(i, r, d); vs[r][d] = x; });
    __syncthreads();
    const int cnt = min(kF32Rows, a.n_k - m0);
    for (int r = lane; r < cnt; r += kF32Lanes) {
      const float s = dot_f32<D>(qr, ks[r]);
      const float dp = dot_f32<D>(gr, vs[r]);
      const float ds = expf(s * a.scale - lse) * (dp + dl);   // dl = -Delta
#pragma unroll
      for (int d = 0; d < D; ++d) dq[d] = fmaf(ds, ks[r][d], dq[d]);
    }
  }
  sum_lanes<D>(dq);
  if (!ok) return;
#pragma unroll
  for (int d = 0; d < D; ++d)
    if (d % kF32Lanes == lane) reinterpret_cast<float*>(a.dq)[qrow + d] = dq[d] * a.scale;
}

// Launches a float32 kernel of kF32Out output rows per workgroup over `rows`
// rows per batch-head, in as many launches as keep each at most 2^31 work-items.
template <typename K>
hipError_t launch_f32_rows(K kernel, BwdArgs a, int rows, hipStream_t stream) {
  const int64_t per_bh = (rows + kF32Out - 1) / kF32Out;
  const int64_t max_bh = std::max<int64_t>(1, (int64_t(1) << 31) / (per_bh * kF32Threads));
  for (int64_t b0 = 0; b0 < a.BH; b0 += max_bh) {
    BwdArgs c = a;
    c.bh0 = static_cast<int>(b0);
    const int64_t nb = std::min<int64_t>(max_bh, a.BH - b0);
    kernel<<<dim3(static_cast<unsigned>(per_bh * nb)), kF32Threads, 0, stream>>>(c);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// ---------------------------------------------------------------- dispatch

constexpr int kWavesBwd = 4;

// Direct staging needs head dim 32..128 and every batch-head's rows under
// 2 GB (32-bit buffer offsets).
bool bwd_direct(int D, int n_q, int n_k) {
  const int64_t n = n_q > n_k ? n_q : n_k;
  return D >= 32 && n * D * 2 < (int64_t(1) << 31);
}

// The direct-staged dQ and dK/dV launches (head dims 32..128; false for 16).
// The dQ kernel goes first: it also stores -Delta and LSE * log2(e), which
// the dK/dV kernel reads.
template <int D>
typename std::enable_if<(D >= 32), bool>::type launch_direct(const BwdArgs& kv, dim3 grid_kv, const BwdArgs& qa,
                                                              dim3 grid_q, hipStream_t stream) {
  if (!bwd_direct(D, kv.n_q, kv.n_k)) return false;
  bwd_dq_direct<D, kWavesBwd><<<grid_q, kWavesBwd * 64, 0, stream>>>(qa);
  bwd_dkdv_direct<D, kWavesBwd><<<grid_kv, kWavesBwd * 64, 0, stream>>>(kv);
  return true;
}
template <int D>
typename std::enable_if<(D < 32), bool>::type launch_direct(const BwdArgs&, dim3, const BwdArgs&, dim3,
                                                             hipStream_t) {
  return false;
}

template <int D>
hipError_t run(BwdArgs a, bool bf16, hipStream_t stream) {
  const int64_t rows = static_cast<int64_t>(a.BH) * a.n_q;
  const dim3 grid_delta(static_cast<unsigned>((rows + 255) / 256));
  if (bf16) {
    BwdArgs kv = a;
    kv.tiles = (a.n_k + 32 * kWavesBwd - 1) / (32 * kWavesBwd);
    const dim3 grid_kv(static_cast<unsigned>(a.BH) * kv.tiles);
    BwdArgs qa = a;
    qa.tiles = (a.n_q + 32 * kWavesBwd - 1) / (32 * kWavesBwd);
    const dim3 grid_q(static_cast<unsigned>(a.BH) * qa.tiles);
    if (launch_direct<D>(kv, grid_kv, qa, grid_q, stream)) return hipGetLastError();
    bwd_delta<D, true><<<grid_delta, 256, 0, stream>>>(a);
    bwd_dkdv_bf16<D, kWavesBwd><<<grid_kv, kWavesBwd * 64, 0, stream>>>(kv);
    bwd_dq_bf16<D, kWavesBwd><<<grid_q, kWavesBwd * 64, 0, stream>>>(qa);
  } else {
    bwd_delta<D, false><<<grid_delta, 256, 0, stream>>>(a);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) e = launch_f32_rows(bwd_dkdv_f32<D>, a, a.n_k, stream);
    if (e == hipSuccess) e = launch_f32_rows(bwd_dq_f32<D>, a, a.n_q, stream);
    return e;
  }
  return hipGetLastError();
}

}  // namespace

// Scratch of fa2_bwd_noalloc: the -Delta and LSE*log2(e) rows the dK/dV and dQ kernels read,
// in device memory that the code object itself holds, so that the entry
// point allocates nothing. Every GPU the library runs on holds its own copy
// until the process ends; every call on one GPU shares it.
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

namespace {

// Device address of `scratch` per device, looked up once with that device
// current. In host code `scratch` names a host-side stand-in, not the device
// array: only the looked-up address is passed to kernels.
std::mutex g_scratch_mu;
std::atomic<float*> g_scratch_addr[64];

hipError_t scratch_address(float** out) {
  int dev = 0;
  const hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  float* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      void* a = nullptr;
      const hipError_t e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      p = static_cast<float*>(a);
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

hipError_t init_device() {
  float* p = nullptr;
  return scratch_address(&p);
}

hipError_t launch_fa2_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                                  const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                  int BH, int n_q, int n_k, int D, float scale, bool bf16,
                                  hipStream_t stream) {
  if (static_cast<int64_t>(BH) * n_q * static_cast<int64_t>(2 * sizeof(float)) >
      static_cast<int64_t>(kNoAllocScratchBytes))
    return hipErrorInvalidValue;
  float* ws = nullptr;
  const hipError_t err = scratch_address(&ws);
  if (err != hipSuccess) return err;
  return launch_fa2_bwd(q, k, v, o, dout, lse, dq, dk, dv, ws, BH, n_q, n_k, D, scale, bf16,
                        stream);
}

hipError_t launch_fa2_bwd(const void* q, const void* k, const void* v, const void* o,
                          const void* dout, const float* lse, void* dq, void* dk, void* dv,
                          float* workspace, int BH, int n_q, int n_k, int D, float scale, bool bf16,
                          hipStream_t stream) {
  float* delta = workspace;
  float* lse2 = workspace + static_cast<int64_t>(BH) * n_q;
  BwdArgs a{static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
            static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(o),
            static_cast<const uint16_t*>(dout), lse, static_cast<uint16_t*>(dq),
            static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv), delta, lse2, BH, n_q, n_k, 0,
            scale, scale * kLog2e};
  switch (D) {
    case 16: return run<16>(a, bf16, stream);
    case 32: return run<32>(a, bf16, stream);
    case 64: return run<64>(a, bf16, stream);
    case 128: return run<128>(a, bf16, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace psa
