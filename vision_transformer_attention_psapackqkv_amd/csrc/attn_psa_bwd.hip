// PSA backward for gfx950: the gradient of the fused PSA forward with respect
// to the NCHW QKV tensor, computed as one dual-V Flash Attention 2 backward.
//
// vision-rs book, "Custom Kernels", sections "Position-Sensitive Attention
// (PSA)" and "Flash Attention 2". The forward's output is [O_lo | O_hi] with
// O_j = softmax(s Q K^T) V_j, plus the V residual (a copy of the V channels).
// Both halves share P = softmax(s Q K^T), so with V = [V_lo | V_hi] and
// dO = [dO_lo | dO_hi] (value width DV = 2*KEY_DIM) the sum over the halves
// of each half's FA2 backward is one backward of width DV:
//   Delta = rowsum(dO * O)             (over both halves)
//   dS    = P * (dO V^T - Delta)       (one dS serves both halves)
//   dV    = P^T dO + dV_residual,   dK = s dS^T Q,   dQ = s dS K.
// Like the page's FA2 backward, dQ and dK/dV are separate kernels with their
// own grids (no atomics), launched in this order:
//   psa_bwd_dq:   one workgroup per (bh, 128 queries), looping over 64-key tiles;
//                 it also stores -Delta and LSE * log2(e) for its pixels;
//   psa_bwd_dkdv: one workgroup per (bh, 128 keys), looping over 64-query tiles.
// Every tensor is read and written in NCHW (channel rows of N pixels), so the
// split, pack and unpack permutations of an unfused chain never run.
//
// dK/dV kernel, per wave (32 keys) and 32-query block; the wave's K and V rows
// are register operands:
//   S [q][key] = Q K^T          A = Q  (LDS [d][q] tile, transposed read)
//   dP[q][key] = dO V^T         A = dO (LDS [dv][q] tile, transposed read)
//   dV^T[dv][key] += dO^T P     A = dO^T (LDS, 16-byte read), B = P (registers)
//   dK^T[d][key]  += Q^T dS     A = Q^T  (LDS, 16-byte read), B = dS (registers)
// dQ kernel, per wave (32 queries) and 32-key block; Q and dO rows in registers:
//   S^T [key][q] = K Q^T        A = K (LDS [d][key] tile, transposed read)
//   dP^T[key][q] = V dO^T       A = V (LDS [dv][key] tile, transposed read)
//   dQ^T[d][q]  += K^T dS^T     A = K^T (LDS, 16-byte read), B = dS^T (registers)
// The transposed reads permute the rows of the first products (key_of_row), so
// the accumulator a lane holds is directly the B operand of the last product.
// LDS tiles are unpadded rows of 64 pixels with XOR-swizzled 16-byte chunks
// (tile_chunk_pos), read both ways; they are filled straight from global memory
// (buffer loads with an LDS destination) when N is a multiple of 8, through registers
// otherwise. Scores use base 2: P = 2^(S * s*log2(e) - LSE*log2(e)).
//
// float32 (PSA_F32): four lanes per row on the VALU, in float32 with expf, one
// V half at a time. Delta, dS, dQ and dK are linear over the halves (Delta =
// Delta_lo + Delta_hi, dS = dS_lo + dS_hi with dS_j = P * (dO_j V_j^T -
// Delta_j)), so each half runs a Delta pass, a dK/dV pass and a dQ pass, and
// the second half adds its dQ and dK to the first's.
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "psa_device.hpp"
#include "psa_launch.hpp"

namespace psa {
namespace {

constexpr int kTN = 64;        // pixels per LDS tile (queries or keys)
constexpr int kWavesBwd = 4;   // 32 rows (keys or queries) per wave
constexpr int kThreadsBwd = kWavesBwd * 64;

struct PsaBwdArgs {
  const uint16_t* qkv;    // [BH * 4KD, N]: per head Q, K, V_lo, V_hi channel rows
  const uint16_t* o;      // [BH * DV, N]
  const uint16_t* dout;   // [BH * DV, N]
  const uint16_t* dvres;  // [BH * DV, N] or null
  const float* lse;       // [BH, N], natural log
  float* delta;           // -Delta = -rowsum(dO O) over both halves, [BH, N]
  float* lse2;            // [BH, N]: LSE * log2(e)
  uint16_t* dqkv;         // [BH * 4KD, N]
  int BH, N, tiles;       // tiles: workgroups per batch-head
  float scale, c;         // s and s * log2(e)
};

// blockIdx -> (bh, tile) with each XCD given a contiguous run of tiles
// (workgroups are dispatched round-robin over the 8 XCDs).
__device__ __forceinline__ void xcd_tile(int total, int tiles, int& bh, int& t) {
  const int i = blockIdx.x;
  const int per = total / 8;
  const int L = (i < per * 8) ? (i % 8) * per + i / 8 : i;
  bh = L / tiles;
  t = L - bh * tiles;
}

// Element (row, col) of a swizzled [rows][64] LDS tile.
__device__ __forceinline__ const uint16_t* tile_at(const uint16_t* tile, int row, int col) {
  return tile + row * kTN + tile_chunk_pos(row, col >> 3) * 8 + (col & 7);
}

// One operand of 8 values down rows r0 .. r0+7 at column col of a swizzled tile:
// two ds_read_b64_tr_b16 (rows r0.. and r0+4..), see lds_read_tr8.
__device__ __forceinline__ bf16x8 tile_read_tr8(const uint16_t* tile, int r0, int col) {
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)tile_at(tile, r0, col));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)tile_at(tile, r0 + 4, col));
  const u32x2 x = __builtin_bit_cast(u32x2, lo), y = __builtin_bit_cast(u32x2, hi);
  return as_bf16x8(u32x4{x[0], x[1], y[0], y[1]});
}

// 8 consecutive columns (one 16-byte chunk) of row `row` of a swizzled tile.
__device__ __forceinline__ bf16x8 tile_read8(const uint16_t* tile, int row, int chunk) {
  return *reinterpret_cast<const bf16x8*>(tile + row * kTN + tile_chunk_pos(row, chunk) * 8);
}

// Rows [0, R) x pixels [m0, m0 + 64) of an NCHW slab (row r at src + r*N) into a
// swizzled LDS tile, straight from global memory: wave instruction b fills the
// 1 KB of rows 8b .. 8b+7, lane i the i-th 16-byte chunk, fetching the pixel
// chunk the swizzle puts there. Buffer loads over the R x N slab (under 2 GB:
// the launcher checks): the lane's offset inside its block does not depend on
// m0, and the block's origin is a scalar offset. Pixels past N repeat real
// data (the kernels give them zero weight). Needs N a multiple of 8.
template <int R>
__device__ __forceinline__ void stage_direct(const uint16_t* src, int N, int m0, int wave, int lane,
                                             uint16_t* dst) {
  constexpr int BLOCKS = R / 8;
  static_assert(R % 8 == 0, "whole 1 KB blocks");
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(src), 0, R * N * 2, kBufferWord3);
  const bool last = m0 + kTN > N;
  if (!last) {
    // Whole tile: the lane's offset depends on the lane and block only (the
    // compiler keeps it across tiles); the tile origin goes in the scalar offset.
#pragma unroll
    for (int i = 0; i < (BLOCKS + kWavesBwd - 1) / kWavesBwd; ++i) {
      const int b = wave + i * kWavesBwd;
      if (BLOCKS % kWavesBwd != 0 && b >= BLOCKS) break;
      const int r = lane >> 3;
      const int pos = tile_chunk_pos(b * 8 + r, lane & 7) * 8;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsrc, (__attribute__((address_space(3))) void*)(dst + b * 512), 16,
          static_cast<uint32_t>(r * N + pos) * 2u, (b * 8 * N + m0) * 2, 0, 0);
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < (BLOCKS + kWavesBwd - 1) / kWavesBwd; ++i) {
    const int b = wave + i * kWavesBwd;
    if (BLOCKS % kWavesBwd != 0 && b >= BLOCKS) break;
    const int r = lane >> 3;
    const int pos = tile_chunk_pos(b * 8 + r, lane & 7) * 8;
    const int m = m0 + pos < N ? m0 + pos : N - 8;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsrc, (__attribute__((address_space(3))) void*)(dst + b * 512), 16,
        static_cast<uint32_t>(r * N + m) * 2u, b * 8 * N * 2, 0, 0);
  }
}

// The same tile through registers, for any N (pixels past N read as zero).
template <int R>
struct StageRegs {
  static constexpr int CH = R * 8;   // 16-byte chunks
  static constexpr int PER = (CH + kThreadsBwd - 1) / kThreadsBwd;
  u32x4 r[PER];

  __device__ __forceinline__ void load(const uint16_t* src, int N, int m0, int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = tid + i * kThreadsBwd;
      if (c < CH) {
        const int row = c >> 3;
        const int m = m0 + tile_chunk_pos(row, c & 7) * 8;
        r[i] = gather8(src + static_cast<int64_t>(row) * N + m, 1, m, N);
      }
    }
  }
  __device__ __forceinline__ void store(uint16_t* dst, int tid) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = tid + i * kThreadsBwd;
      if (c < CH) *reinterpret_cast<u32x4*>(dst + c * 8) = r[i];
    }
  }
};

// ---------------------------------------------------------------- dK / dV

template <int KD, bool kVecN, int kOcc>
__global__ __launch_bounds__(kThreadsBwd, kOcc) void psa_bwd_dkdv(PsaBwdArgs a) {
  constexpr int DV = 2 * KD;
  constexpr int DP = KD < 32 ? 32 : KD;   // Q tile rows (one MFMA block minimum)
  constexpr int NDS = KD / 16, NVS = DV / 16;
  constexpr int NDK = DP / 32, NDV = DV / 32;
  constexpr int kQbUnroll = KD <= 32 && kVecN ? kTN / 32 : 1;   // query blocks unrolled per tile
  constexpr int Q_EL = DP * kTN, DO_EL = DV * kTN;
  constexpr int BUF = Q_EL + DO_EL + 2 * kTN * 2;   // + LSE*log2(e) and -Delta (floats)
  // Two tile buffers as two objects reached through restrict pointers, so the
  // LDS reads of one tile need not wait for the direct loads into the other.
  __shared__ __attribute__((aligned(16))) uint16_t smem0[BUF];
  __shared__ __attribute__((aligned(16))) uint16_t smem1[BUF];

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i16 = lane & 15, t16 = (lane >> 4) & 1;
  const int N = a.N;
  int bh, kt;
  xcd_tile(a.BH * a.tiles, a.tiles, bh, kt);
  const int key = kt * 32 * kWavesBwd + wave * 32 + l32;
  const bool k_ok = key < N;
  const uint16_t* qkv = a.qkv + static_cast<int64_t>(bh) * 4 * KD * N;
  const uint16_t* dout = a.dout + static_cast<int64_t>(bh) * DV * N;

  if constexpr (DP > KD) {   // Q tile rows KD..DP-1 stay zero
    for (int e = tid; e < (DP - KD) * kTN; e += kThreadsBwd) {
      smem0[KD * kTN + e] = 0;
      smem1[KD * kTN + e] = 0;
    }
  }

  // B operands of S and dP: K[key][16ds + 8g + j] and V[key][16vs + 8g + j].
  // Keys past N load pixel N - 1 (every load unconditional, all in flight
  // together) and are zeroed afterwards.
  bf16x8 kop[NDS], vop[NVS];
  {
    const int kc = min(key, N - 1);
    u32x4 kr[NDS], vr[NVS];
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds)
      kr[ds] = gather8(qkv + static_cast<int64_t>(KD + ds * 16 + g * 8) * N + kc, N, 0, 8);
#pragma unroll
    for (int vs = 0; vs < NVS; ++vs)
      vr[vs] = gather8(qkv + static_cast<int64_t>(2 * KD + vs * 16 + g * 8) * N + kc, N, 0, 8);
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) kop[ds] = as_bf16x8(k_ok ? kr[ds] : zero4());
#pragma unroll
    for (int vs = 0; vs < NVS; ++vs) vop[vs] = as_bf16x8(k_ok ? vr[vs] : zero4());
  }
  f32x16 dk[NDK], dv[NDV];
#pragma unroll
  for (int b = 0; b < NDK; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) dk[b][r] = 0.0f;
#pragma unroll
  for (int b = 0; b < NDV; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) dv[b][r] = 0.0f;

  // Per query tile: Q rows, dO rows, and (threads 0..127) LSE*log2(e) / -Delta.
  StageRegs<KD> sq;
  StageRegs<DV> sg;
  float fval = 0.0f;
  auto issue = [&](int t, uint16_t* buf) {
    const int q0 = t * kTN;
    if constexpr (kVecN) {
      stage_direct<KD>(qkv, N, q0, wave, lane, buf);
      stage_direct<DV>(dout, N, q0, wave, lane, buf + Q_EL);
    } else {
      sq.load(qkv, N, q0, tid);
      sg.load(dout, N, q0, tid);
    }
    if (tid < 2 * kTN) {
      const int q = q0 + (tid & (kTN - 1));
      const bool ok = q < N;
      const int64_t i = static_cast<int64_t>(bh) * N + q;
      // queries past N: P = 2^-inf = 0
      fval = tid < kTN ? (ok ? a.lse2[i] : INFINITY) : (ok ? a.delta[i] : 0.0f);
    }
  };
  auto finish = [&](uint16_t* buf) {
    if constexpr (kVecN) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    } else {
      sq.store(buf, tid);
      sg.store(buf + Q_EL, tid);
    }
    if (tid < 2 * kTN) reinterpret_cast<float*>(buf + Q_EL + DO_EL)[tid] = fval;
  };

  const int n_tiles = (N + kTN - 1) / kTN;
  issue(0, smem0);
  finish(smem0);
  __syncthreads();

  // One query tile, read from qs while the next one is loaded into nbuf.
  auto tile = [&](int qt, const uint16_t* __restrict__ qs, uint16_t* __restrict__ nbuf)
                  __attribute__((always_inline)) {
    const uint16_t* gs = qs + Q_EL;
    const float* fl = reinterpret_cast<const float*>(gs + DO_EL);
    const bool more = qt + 1 < n_tiles;
    if (more) issue(qt + 1, nbuf);

    // Up to key_dim 32, with directly staged tiles, the blocks are unrolled
    // (every LDS address a per-lane offset plus a constant) but kept one after
    // the other, not interleaved, which would hold both blocks' registers. The
    // other kernels keep the rolled loop, which spills less or not at all.
#pragma unroll kQbUnroll
    for (int qb = 0; qb < kTN / 32; ++qb) {
      if (kQbUnroll > 1 && qb > 0) __builtin_amdgcn_sched_barrier(0);
      // Rows of S and dP: query qb*32 + 16*(r/8) + 8g + r%8 in element r.
      // dP's accumulator starts at -Delta, so it ends as dP - Delta.
      const int col = qb * 32 + 16 * t16 + tr_key_col(i16 & 3);
      f32x16 sacc, pacc;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int q = qb * 32 + 16 * h + 8 * g;
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(fl + kTN + q);
        const f32x4 d1 = *reinterpret_cast<const f32x4*>(fl + kTN + q + 4);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          sacc[8 * h + j] = 0.0f;
          pacc[8 * h + j] = j < 4 ? d0[j] : d1[j - 4];   // -Delta
        }
      }
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds)
        sacc = mfma32x32x16(tile_read_tr8(qs, ds * 16 + 8 * g + (i16 >> 2), col), kop[ds], sacc);
#pragma unroll
      for (int vs = 0; vs < NVS; ++vs)
        pacc = mfma32x32x16(tile_read_tr8(gs, vs * 16 + 8 * g + (i16 >> 2), col), vop[vs], pacc);
      bf16x8 pb[2], sb[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int q = qb * 32 + 16 * h + 8 * g;
        const f32x4 l0 = *reinterpret_cast<const f32x4*>(fl + q);
        const f32x4 l1 = *reinterpret_cast<const f32x4*>(fl + q + 4);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int r = 8 * h + j;
          const float p = fast_exp2(fmaf(sacc[r], a.c, -(j < 4 ? l0[j] : l1[j - 4])));
          pb[h][j] = static_cast<__bf16>(p);
          sb[h][j] = static_cast<__bf16>(p * pacc[r]);
        }
      }
      // dV^T += dO^T P and dK^T += Q^T dS over the block's queries, 16 per step.
#pragma unroll
      for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int b = 0; b < NDV; ++b)
          dv[b] = mfma32x32x16(tile_read8(gs, b * 32 + l32, 4 * qb + 2 * s + g), pb[s], dv[b]);
#pragma unroll
        for (int b = 0; b < NDK; ++b)
          dk[b] = mfma32x32x16(tile_read8(qs, b * 32 + l32, 4 * qb + 2 * s + g), sb[s], dk[b]);
      }
    }
    if (more) finish(nbuf);
    __syncthreads();
  };
  // A wave whose 32 keys all lie past N (the last key tile of a batch-head when
  // N is not a multiple of 128) only helps stage the tiles and meets the
  // barriers, in a loop of its own (a branch inside the loop below would cost
  // it registers).
  if (kt * 32 * kWavesBwd + wave * 32 >= N) {
    for (int t = 0; t < n_tiles; ++t) {
      if (t + 1 < n_tiles) {
        uint16_t* nb = (t & 1) ? smem0 : smem1;
        issue(t + 1, nb);
        finish(nb);
      }
      __syncthreads();
    }
    return;
  }
  for (int qt = 0; qt < n_tiles; ++qt) {   // tile t lives in smem0 for even t, smem1 for odd
    const bool odd = qt & 1;
    tile(qt, odd ? smem1 : smem0, odd ? smem0 : smem1);
  }

  if (!k_ok) return;
  uint16_t* dq_out = a.dqkv + static_cast<int64_t>(bh) * 4 * KD * N;
  // dK^T / dV^T element r: row 32b + 8(r/4) + 4g + r%4, column = this lane's key.
#pragma unroll
  for (int b = 0; b < NDK; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int d = b * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
      if (d < KD) dq_out[static_cast<int64_t>(KD + d) * N + key] = float_to_bf16_bits(dk[b][r] * a.scale);
    }
  const uint16_t* dvres = a.dvres ? a.dvres + static_cast<int64_t>(bh) * DV * N : nullptr;
#pragma unroll
  for (int b = 0; b < NDV; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int d = b * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
      float x = dv[b][r];
      if (dvres) x += bf16_bits_to_float(dvres[static_cast<int64_t>(d) * N + key]);
      dq_out[static_cast<int64_t>(2 * KD + d) * N + key] = float_to_bf16_bits(x);
    }
}

// ---------------------------------------------------------------- dQ

template <int KD, bool kVecN, int kOcc>
__global__ __launch_bounds__(kThreadsBwd, kOcc) void psa_bwd_dq(PsaBwdArgs a) {
  constexpr int DV = 2 * KD;
  constexpr int DP = KD < 32 ? 32 : KD;   // K tile rows (one MFMA block minimum)
  constexpr int NDS = KD / 16, NVS = DV / 16, NDB = DP / 32;
  constexpr int K_EL = DP * kTN, V_EL = DV * kTN;
  constexpr int BUF = K_EL + V_EL;
  // Two tile buffers as two objects reached through restrict pointers, so the
  // LDS reads of one tile need not wait for the direct loads into the other.
  __shared__ __attribute__((aligned(16))) uint16_t smem0[BUF];
  __shared__ __attribute__((aligned(16))) uint16_t smem1[BUF];

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i16 = lane & 15, t16 = (lane >> 4) & 1;
  const int N = a.N;
  int bh, qt;
  xcd_tile(a.BH * a.tiles, a.tiles, bh, qt);
  const int q = qt * 32 * kWavesBwd + wave * 32 + l32;
  const bool q_ok = q < N;
  const uint16_t* qkv = a.qkv + static_cast<int64_t>(bh) * 4 * KD * N;
  const uint16_t* dout = a.dout + static_cast<int64_t>(bh) * DV * N;

  if constexpr (DP > KD) {   // K tile rows KD..DP-1 stay zero
    for (int e = tid; e < (DP - KD) * kTN; e += kThreadsBwd) {
      smem0[KD * kTN + e] = 0;
      smem1[KD * kTN + e] = 0;
    }
  }

  // B operands: Q[q][16ds + 8g + j] and dO[q][16vs + 8g + j]. Queries past N
  // load pixel N - 1 (every load unconditional, all in flight together) and
  // are zeroed afterwards.
  // This kernel runs first and also computes, for its pixels, -Delta =
  // -rowsum(dO o O) over both halves (lanes l and l ^ 32 each hold half of the
  // channels) and LSE * log2(e), and stores both for the dK/dV kernel.
  bf16x8 qop[NDS], gop[NVS];
  float l2, dl;
  {
    const int qc = min(q, N - 1);
    const int64_t row = static_cast<int64_t>(bh) * N + qc;
    const uint16_t* out = a.o + static_cast<int64_t>(bh) * DV * N;
    u32x4 qr[NDS], gr[NVS], orow[NVS];
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds)
      qr[ds] = gather8(qkv + static_cast<int64_t>(ds * 16 + g * 8) * N + qc, N, 0, 8);
#pragma unroll
    for (int vs = 0; vs < NVS; ++vs) {
      gr[vs] = gather8(dout + static_cast<int64_t>(vs * 16 + g * 8) * N + qc, N, 0, 8);
      orow[vs] = gather8(out + static_cast<int64_t>(vs * 16 + g * 8) * N + qc, N, 0, 8);
    }
    const float lv = a.lse[row] * kLog2e;
    float part = 0.0f;
#pragma unroll
    for (int vs = 0; vs < NVS; ++vs)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        part = fmaf(__builtin_bit_cast(float, orow[vs][w] << 16), __builtin_bit_cast(float, gr[vs][w] << 16), part);
        part = fmaf(__builtin_bit_cast(float, orow[vs][w] & 0xFFFF0000u),
                    __builtin_bit_cast(float, gr[vs][w] & 0xFFFF0000u), part);
      }
    const float dv = -(part + __shfl_xor(part, 32));
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) qop[ds] = as_bf16x8(q_ok ? qr[ds] : zero4());
#pragma unroll
    for (int vs = 0; vs < NVS; ++vs) gop[vs] = as_bf16x8(q_ok ? gr[vs] : zero4());
    l2 = q_ok ? lv : INFINITY;
    dl = q_ok ? dv : 0.0f;
    if (q_ok && g == 0) {
      a.delta[row] = dv;
      a.lse2[row] = lv;
    }
  }
  f32x16 dq[NDB];
#pragma unroll
  for (int b = 0; b < NDB; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[b][r] = 0.0f;

  StageRegs<KD> sk;
  StageRegs<DV> sv;
  auto issue = [&](int t, uint16_t* buf) {
    if constexpr (kVecN) {
      stage_direct<KD>(qkv + static_cast<int64_t>(KD) * N, N, t * kTN, wave, lane, buf);
      stage_direct<DV>(qkv + static_cast<int64_t>(2 * KD) * N, N, t * kTN, wave, lane, buf + K_EL);
    } else {
      sk.load(qkv + static_cast<int64_t>(KD) * N, N, t * kTN, tid);
      sv.load(qkv + static_cast<int64_t>(2 * KD) * N, N, t * kTN, tid);
    }
  };
  auto finish = [&](uint16_t* buf) {
    if constexpr (kVecN) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    } else {
      sk.store(buf, tid);
      sv.store(buf + K_EL, tid);
    }
  };

  const int n_tiles = (N + kTN - 1) / kTN;
  issue(0, smem0);
  finish(smem0);
  __syncthreads();

  // One key tile, read from ks while the next one is loaded into nbuf. Only
  // the last tile (`last` true) can hold keys past N, and only its code masks
  // them: a run-time test on every tile is flattened by the compiler into a
  // compare and a select per score.
  auto tile = [&](int kt, const uint16_t* __restrict__ ks, uint16_t* __restrict__ nbuf, auto last)
                  __attribute__((always_inline)) {
    const uint16_t* vs_ = ks + K_EL;
    const bool more = kt + 1 < n_tiles;
    if (more) issue(kt + 1, nbuf);

    bf16x8 sb[kTN / 16];   // dS^T, 16 keys per step
#pragma unroll
    for (int kb = 0; kb < kTN / 32; ++kb) {
      // Rows of S^T and dP^T: key kb*32 + 16*(r/8) + 8g + r%8 in element r.
      // dP^T's accumulator starts at -Delta, so it ends as dP^T - Delta.
      const int col = kb * 32 + 16 * t16 + tr_key_col(i16 & 3);
      f32x16 sacc, pacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sacc[r] = 0.0f;
        pacc[r] = dl;   // -Delta
      }
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds)
        sacc = mfma32x32x16(tile_read_tr8(ks, ds * 16 + 8 * g + (i16 >> 2), col), qop[ds], sacc);
#pragma unroll
      for (int vs = 0; vs < NVS; ++vs)
        pacc = mfma32x32x16(tile_read_tr8(vs_, vs * 16 + 8 * g + (i16 >> 2), col), gop[vs], pacc);
      // Keys past N get P = 0.
      if constexpr (decltype(last)::value) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kt * kTN + kb * 32 + 16 * (r >> 3) + 8 * g + (r & 7) >= N) sacc[r] = -INFINITY;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(fmaf(sacc[r], a.c, -l2));
        sb[kb * 2 + (r >> 3)][r & 7] = static_cast<__bf16>(p * pacc[r]);
      }
    }
    // dQ^T += K^T dS^T over the tile's keys, 16 per step.
#pragma unroll
    for (int s = 0; s < kTN / 16; ++s)
#pragma unroll
      for (int b = 0; b < NDB; ++b) dq[b] = mfma32x32x16(tile_read8(ks, b * 32 + l32, 2 * s + g), sb[s], dq[b]);

    if (more) finish(nbuf);
    __syncthreads();
  };
  // A wave whose 32 queries all lie past N only helps stage the tiles, as in
  // the dK/dV kernel.
  if (qt * 32 * kWavesBwd + wave * 32 >= N) {
    for (int t = 0; t < n_tiles; ++t) {
      if (t + 1 < n_tiles) {
        uint16_t* nb = (t & 1) ? smem0 : smem1;
        issue(t + 1, nb);
        finish(nb);
      }
      __syncthreads();
    }
    return;
  }
  // Tile t lives in smem0 for even t, smem1 for odd. Two tiles per trip, so
  // that each reads a fixed LDS object and every LDS address is a
  // loop-invariant per-lane offset plus a constant (-1.1 % on the 40x40 map;
  // the dK/dV kernel, where the same change costs registers it lacks, keeps
  // one tile per trip). The last tile masks keys past N.
  int kt = 0;
  for (; kt + 2 < n_tiles; kt += 2) {
    tile(kt, smem0, smem1, std::false_type{});
    tile(kt + 1, smem1, smem0, std::false_type{});
  }
  if (kt + 1 < n_tiles) {
    tile(kt, smem0, smem1, std::false_type{});
    tile(kt + 1, smem1, smem0, std::true_type{});
  } else {
    tile(kt, smem0, smem1, std::true_type{});
  }

  if (!q_ok) return;
  uint16_t* dq_out = a.dqkv + static_cast<int64_t>(bh) * 4 * KD * N;
#pragma unroll
  for (int b = 0; b < NDB; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int d = b * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
      if (d < KD) dq_out[static_cast<int64_t>(d) * N + q] = float_to_bf16_bits(dq[b][r] * a.scale);
    }
}

// ---------------------------------------------------------------- float32

struct PsaBwdF32Args {
  const float* qkv;    // [BH * 4KD, N]
  const float* o;      // [BH * DV, N]
  const float* dout;   // [BH * DV, N]
  const float* dvres;  // [BH * DV, N] or null
  const float* lse;    // [BH, N], natural log
  float* delta;        // [BH, N]: -Delta_j of the current half
  float* dqkv;         // [BH * 4KD, N]
  int BH, N, KD, j;    // j: the V half (0: lo, 1: hi)
  float scale;
  int bh0;             // first batch-head of this launch
};

constexpr int kF32Threads = 128;
constexpr int kF32Rows = 32;                        // rows per LDS tile
constexpr int kF32Lanes = 4;                        // lanes per output pixel
constexpr int kF32Out = kF32Threads / kF32Lanes;    // output pixels per workgroup

// Thread element i of a [kF32Rows][cols] LDS tile filled from channel rows:
// pixels (tile rows) fastest, as they are contiguous in NCHW.
__device__ __forceinline__ void f32_rc(int i, int& r, int& d) {
  const int e = static_cast<int>(threadIdx.x) + i * kF32Threads;
  r = e % kF32Rows;
  d = e / kF32Rows;
}

// Adds the partial sums x[0..D) of the four lanes of an output pixel (lanes
// 4i..4i+3); every lane ends with the total.
template <int D>
__device__ __forceinline__ void sum_lanes(float (&x)[D]) {
#pragma unroll
  for (int m = 1; m < kF32Lanes; m <<= 1)
#pragma unroll
    for (int d = 0; d < D; ++d) x[d] += __shfl_xor(x[d], m);
}

// -Delta_j = -sum over half j's channels of dO * O, one thread per pixel.
__global__ __launch_bounds__(256) void psa_bwd_delta_f32(PsaBwdF32Args a) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= static_cast<int64_t>(a.BH) * a.N) return;
  const int bh = static_cast<int>(i / a.N);
  const int n = static_cast<int>(i - static_cast<int64_t>(bh) * a.N);
  const int64_t base = (static_cast<int64_t>(bh) * 2 * a.KD + a.j * a.KD) * a.N + n;
  float s = 0.0f;
#pragma unroll 8
  for (int c = 0; c < a.KD; ++c) s = fmaf(a.dout[base + static_cast<int64_t>(c) * a.N], a.o[base + static_cast<int64_t>(c) * a.N], s);
  a.delta[i] = -s;
}

// dK (summed over the halves) and dV_j: four lanes per key, lane l taking queries
// l, l+4, ... of each tile staged through LDS; the lanes' partial sums are added
// at the end.
template <int KD>
__global__ __launch_bounds__(kF32Threads) void psa_bwd_dkdv_f32(PsaBwdF32Args a) {
  __shared__ float qs[kF32Rows][KD];
  __shared__ float gs[kF32Rows][KD];
  __shared__ float ls[kF32Rows], dls[kF32Rows];
  const int N = a.N;
  const int blocks = (N + kF32Out - 1) / kF32Out;
  const int bh = a.bh0 + static_cast<int>(blockIdx.x / blocks);
  const int lane = threadIdx.x % kF32Lanes;
  const int m = (blockIdx.x % blocks) * kF32Out + threadIdx.x / kF32Lanes;
  const bool ok = m < N;
  const int mc = ok ? m : 0;
  const float* Q = a.qkv + static_cast<int64_t>(bh) * 4 * KD * N;   // channel rows of this head
  const float* G = a.dout + (static_cast<int64_t>(bh) * 2 + a.j) * KD * N;
  float kr[KD], vr[KD], dk[KD], dv[KD];
#pragma unroll
  for (int d = 0; d < KD; ++d) {
    kr[d] = Q[static_cast<int64_t>(KD + d) * N + mc];
    vr[d] = Q[static_cast<int64_t>((2 + a.j) * KD + d) * N + mc];
    dk[d] = dv[d] = 0.0f;
  }
  for (int q0 = 0; q0 < N; q0 += kF32Rows) {
    __syncthreads();
    move_batched<kF32Rows * KD / kF32Threads>(
        [&](int i) { int r, d; f32_rc(i, r, d); return q0 + r < N ? Q[static_cast<int64_t>(d) * N + q0 + r] : 0.0f; },
        [&](int i, float x) { int r, d; f32_rc(i, r, d); qs[r][d] = x; });
    move_batched<kF32Rows * KD / kF32Threads>(
        [&](int i) { int r, d; f32_rc(i, r, d); return q0 + r < N ? G[static_cast<int64_t>(d) * N + q0 + r] : 0.0f; },
        [&](int i, float x) { int r, d; f32_rc(i, r, d); gs[r][d] = x; });
    if (threadIdx.x < kF32Rows) {
      const int r = threadIdx.x;
      const bool in = q0 + r < N;
      ls[r] = in ? a.lse[static_cast<int64_t>(bh) * N + q0 + r] : 0.0f;
      dls[r] = in ? a.delta[static_cast<int64_t>(bh) * N + q0 + r] : 0.0f;
    }
    __syncthreads();
    const int cnt = min(kF32Rows, N - q0);
    for (int r = lane; r < cnt; r += kF32Lanes) {
      const float sc = dot_f32<KD>(qs[r], kr);
      const float dp = dot_f32<KD>(gs[r], vr);
      const float p = expf(sc * a.scale - ls[r]);
      const float ds = p * (dp + dls[r]);   // dls holds -Delta_j
#pragma unroll
      for (int d = 0; d < KD; ++d) {
        dv[d] = fmaf(p, gs[r][d], dv[d]);
        dk[d] = fmaf(ds, qs[r][d], dk[d]);
      }
    }
  }
  sum_lanes<KD>(dk);
  sum_lanes<KD>(dv);
  if (!ok) return;
  // This lane stores the channels d = lane (mod 4).
  auto mine = [&](int d) { return d % kF32Lanes == lane; };
  float* out = a.dqkv + static_cast<int64_t>(bh) * 4 * KD * N;
  const float* res = a.dvres ? a.dvres + (static_cast<int64_t>(bh) * 2 + a.j) * KD * N : nullptr;
  float* pk = out + static_cast<int64_t>(KD) * N + m;             // dK channel rows
  float* pv = out + static_cast<int64_t>(2 + a.j) * KD * N + m;   // dV_j channel rows
  if (a.j == 0) {
#pragma unroll
    for (int d = 0; d < KD; ++d)
      if (mine(d)) pk[static_cast<int64_t>(d) * N] = dk[d] * a.scale;
  } else {
    move_batched<KD>([&](int d) { return mine(d) ? pk[static_cast<int64_t>(d) * N] : 0.0f; },
                     [&](int d, float x) { if (mine(d)) pk[static_cast<int64_t>(d) * N] = x + dk[d] * a.scale; });
  }
  if (res) {
    move_batched<KD>([&](int d) { return mine(d) ? res[static_cast<int64_t>(d) * N + m] : 0.0f; },
                     [&](int d, float x) { if (mine(d)) pv[static_cast<int64_t>(d) * N] = dv[d] + x; });
  } else {
#pragma unroll
    for (int d = 0; d < KD; ++d)
      if (mine(d)) pv[static_cast<int64_t>(d) * N] = dv[d];
  }
}

// dQ (summed over the halves): four lanes per query, lane l taking keys l, l+4,
// ... of each tile staged through LDS; the lanes' partial sums are added at the end.
template <int KD>
__global__ __launch_bounds__(kF32Threads) void psa_bwd_dq_f32(PsaBwdF32Args a) {
  __shared__ float ks[kF32Rows][KD];
  __shared__ float vs[kF32Rows][KD];
  const int N = a.N;
  const int blocks = (N + kF32Out - 1) / kF32Out;
  const int bh = a.bh0 + static_cast<int>(blockIdx.x / blocks);
  const int lane = threadIdx.x % kF32Lanes;
  const int n = (blockIdx.x % blocks) * kF32Out + threadIdx.x / kF32Lanes;
  const bool ok = n < N;
  const int nc = ok ? n : 0;
  const float* Q = a.qkv + static_cast<int64_t>(bh) * 4 * KD * N;
  const float* G = a.dout + (static_cast<int64_t>(bh) * 2 + a.j) * KD * N;
  float qr[KD], gr[KD], dq[KD];
#pragma unroll
  for (int d = 0; d < KD; ++d) {
    qr[d] = Q[static_cast<int64_t>(d) * N + nc];
    gr[d] = G[static_cast<int64_t>(d) * N + nc];
    dq[d] = 0.0f;
  }
  const float lse = a.lse[static_cast<int64_t>(bh) * N + nc];
  const float dl = a.delta[static_cast<int64_t>(bh) * N + nc];   // -Delta_j
  for (int m0 = 0; m0 < N; m0 += kF32Rows) {
    __syncthreads();
    move_batched<kF32Rows * KD / kF32Threads>(
        [&](int i) { int r, d; f32_rc(i, r, d); return m0 + r < N ? Q[static_cast<int64_t>(KD + d) * N + m0 + r] : 0.0f; },
        [&](int i, float x) { int r, d; f32_rc(i, r, d); ks[r][d] = x; });
    move_batched<kF32Rows * KD / kF32Threads>(
        [&](int i) {
          int r, d;
          f32_rc(i, r, d);
          return m0 + r < N ? Q[static_cast<int64_t>((2 + a.j) * KD + d) * N + m0 + r] : 0.0f;
        },
        [&](int i, float x) { int r, d; f32_rc(i, r, d); vs[r][d] = x; });
    __syncthreads();
    const int cnt = min(kF32Rows, N - m0);
    for (int r = lane; r < cnt; r += kF32Lanes) {
      const float sc = dot_f32<KD>(qr, ks[r]);
      const float dp = dot_f32<KD>(gr, vs[r]);
      const float ds = expf(sc * a.scale - lse) * (dp + dl);
#pragma unroll
      for (int d = 0; d < KD; ++d) dq[d] = fmaf(ds, ks[r][d], dq[d]);
    }
  }
  sum_lanes<KD>(dq);
  if (!ok) return;
  auto mine = [&](int d) { return d % kF32Lanes == lane; };   // this lane's channels
  float* p = a.dqkv + static_cast<int64_t>(bh) * 4 * KD * N + n;   // dQ channel rows
  if (a.j == 0) {
#pragma unroll
    for (int d = 0; d < KD; ++d)
      if (mine(d)) p[static_cast<int64_t>(d) * N] = dq[d] * a.scale;
  } else {
    move_batched<KD>([&](int d) { return mine(d) ? p[static_cast<int64_t>(d) * N] : 0.0f; },
                     [&](int d, float x) { if (mine(d)) p[static_cast<int64_t>(d) * N] = x + dq[d] * a.scale; });
  }
}

template <int KD>
hipError_t run_psa_bwd_f32(PsaBwdF32Args a, hipStream_t stream) {
  const int64_t rows = static_cast<int64_t>(a.BH) * a.N;
  const dim3 grid_delta(static_cast<unsigned>((rows + 255) / 256));
  // Batch-heads per launch, so that a launch holds at most 2^31 work-items.
  const int64_t per_bh = (a.N + kF32Out - 1) / kF32Out;
  const int64_t max_bh = std::max<int64_t>(1, (int64_t(1) << 31) / (per_bh * kF32Threads));
  for (int j = 0; j < 2; ++j) {   // the second half adds its dQ and dK to the first's
    a.j = j;
    psa_bwd_delta_f32<<<grid_delta, 256, 0, stream>>>(a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    for (int64_t b0 = 0; b0 < a.BH; b0 += max_bh) {
      PsaBwdF32Args c = a;
      c.bh0 = static_cast<int>(b0);
      const dim3 grid(static_cast<unsigned>(per_bh * std::min<int64_t>(max_bh, a.BH - b0)));
      psa_bwd_dkdv_f32<KD><<<grid, kF32Threads, 0, stream>>>(c);
      psa_bwd_dq_f32<KD><<<grid, kF32Threads, 0, stream>>>(c);
      err = hipGetLastError();
      if (err != hipSuccess) return err;
    }
  }
  return hipSuccess;
}

template <int KD>
hipError_t run_psa_bwd(PsaBwdArgs a, hipStream_t stream) {
  // Workgroups per CU the registers must allow: three up to key_dim 32, two at
  // 64 (the dK/dV kernel walks its two 32-query blocks one after the other to
  // stay in 256 registers); key_dim 128 needs a whole SIMD's register file.
  constexpr int kOccDkdv = KD <= 32 ? 3 : KD <= 64 ? 2 : 1;
  constexpr int kOccDq = KD <= 32 ? 3 : KD <= 64 ? 2 : 1;
  a.tiles = (a.N + 32 * kWavesBwd - 1) / (32 * kWavesBwd);
  const dim3 grid(static_cast<unsigned>(a.BH) * a.tiles);
  // Direct staging addresses one batch-head's [4*KD][N] slab with 32-bit offsets.
  const bool vec_n = a.N % 8 == 0 && static_cast<int64_t>(8) * KD * a.N < (int64_t(1) << 31);
  // dQ first: it stores -Delta and LSE * log2(e), which the dK/dV kernel reads.
  if (vec_n)
    psa_bwd_dq<KD, true, kOccDq><<<grid, kThreadsBwd, 0, stream>>>(a);
  else   // the register-staged tiles need more registers
    psa_bwd_dq<KD, false, KD <= 32 ? 2 : 1><<<grid, kThreadsBwd, 0, stream>>>(a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (vec_n)
    psa_bwd_dkdv<KD, true, kOccDkdv><<<grid, kThreadsBwd, 0, stream>>>(a);
  else   // the register-staged tiles need more registers
    psa_bwd_dkdv<KD, false, KD <= 32 ? 3 : 1><<<grid, kThreadsBwd, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_psa_fused_bwd(const void* qkv, const void* out, const float* lse, const void* dout,
                                const void* dvres, void* dqkv, float* workspace, int BH, int KD,
                                int N, float scale, bool bf16, hipStream_t stream) {
  if (!bf16) {
    PsaBwdF32Args f{static_cast<const float*>(qkv), static_cast<const float*>(out),
                    static_cast<const float*>(dout), static_cast<const float*>(dvres), lse, workspace,
                    static_cast<float*>(dqkv), BH, N, KD, 0, scale};
    switch (KD) {
      case 16: return run_psa_bwd_f32<16>(f, stream);
      case 32: return run_psa_bwd_f32<32>(f, stream);
      case 64: return run_psa_bwd_f32<64>(f, stream);
      case 128: return run_psa_bwd_f32<128>(f, stream);
    }
    return hipErrorInvalidValue;
  }
  PsaBwdArgs a{};
  a.qkv = static_cast<const uint16_t*>(qkv);
  a.o = static_cast<const uint16_t*>(out);
  a.dout = static_cast<const uint16_t*>(dout);
  a.dvres = static_cast<const uint16_t*>(dvres);
  a.lse = lse;
  a.delta = workspace;
  a.lse2 = workspace + static_cast<int64_t>(BH) * N;
  a.dqkv = static_cast<uint16_t*>(dqkv);
  a.BH = BH;
  a.N = N;
  a.scale = scale;
  a.c = scale * kLog2e;
  switch (KD) {
    case 16: return run_psa_bwd<16>(a, stream);
    case 32: return run_psa_bwd<32>(a, stream);
    case 64: return run_psa_bwd<64>(a, stream);
    case 128: return run_psa_bwd<128>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace psa
