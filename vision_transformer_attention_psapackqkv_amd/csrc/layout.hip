// PsaPackQkv, PsaMergeAttn and PsaExtractV for gfx950.
//
// vision-rs book, "Custom Kernels", section "Position-Sensitive Attention
// (PSA)": pack moves the NCHW QKV-conv output [B, 4hKD, H, W] into
// [4, BH, N, KD]; merge and extract move [., BH, N, KD] halves back to NCHW
// [B, 2hKD, H, W]. For one (bh, slot) both sides are contiguous slabs: the NCHW
// side is a [KD, N] matrix (channel rows of N pixels), the packed side an
// [N, KD] matrix. So every op is a batch of [KD, N] <-> [N, KD] transposes
// with a slab-index permutation, and each is bound by HBM bandwidth.
//
// Each thread moves one VEC x VEC block (VEC = 16 bytes / element size):
// VEC 16-byte loads, a transpose in registers, VEC 16-byte stores. Threads are
// laid out with the d-block index fastest, so every load instruction of a
// wave covers whole 128-byte runs of NCHW rows and every store instruction
// whole packed rows. No LDS is needed. Rows whose start is not 16-byte
// aligned (N not a multiple of VEC) take a scalar kernel instead. Measured on
// MI355X at the 80x80 map, 256-thread workgroups suit pack and 128-thread
// workgroups suit merge and extract (both above a plain device copy).
#include "psa_device.hpp"
#include "psa_launch.hpp"

namespace psa {
namespace {

constexpr int kThreads = 256;            // scalar kernel
constexpr int kThreadsToRows = 256;      // pack
constexpr int kThreadsToNchw = 128;      // merge, extract

// 8x8 transpose of 16-bit elements: in[r] holds row r (8 elements, two per
// 32-bit word, element 2w in the low half of word w); out[c] receives column c.
__device__ __forceinline__ void transpose_block(const u32x4 (&in)[8], u32x4 (&out)[8]) {
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

// 4x4 transpose of 32-bit elements.
__device__ __forceinline__ void transpose_block(const u32x4 (&in)[4], u32x4 (&out)[4]) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
#pragma unroll
    for (int w = 0; w < 4; ++w) out[c][w] = in[w][c];
  }
}

struct SlabGeom {
  int BH, KD, N;
  int slots;      // slabs per bh on the NCHW side: 4 for pack, 2 for merge/extract
  int slot0;      // first packed slot touched: 0 for pack and merge, 2 for extract
};

// NCHW-side offset of slab t = bh*slots + s, and packed-side offset of the same slab.
__device__ __forceinline__ void slab_offsets(const SlabGeom& g, int t, int64_t& nchw_off,
                                             int64_t& rows_off) {
  const int bh = t / g.slots;
  const int s = t - bh * g.slots;
  const int64_t slab = static_cast<int64_t>(g.KD) * g.N;
  nchw_off = static_cast<int64_t>(t) * slab;
  rows_off = (static_cast<int64_t>(g.slot0 + s) * g.BH + bh) * slab;
}

// kToRows = true: NCHW [KD, N] slabs -> packed [N, KD] slabs (pack).
// kToRows = false: packed [N, KD] slabs -> NCHW [KD, N] slabs (merge, extract).
template <int kEltBytes, bool kToRows, int kTh = kToRows ? kThreadsToRows : kThreadsToNchw>
__global__ __launch_bounds__(kTh) void transpose_slabs_vec(const void* __restrict__ src_v,
                                                           void* __restrict__ dst_v,
                                                           SlabGeom g, int tiles_per_slab) {
  constexpr int VEC = 16 / kEltBytes;
  const int DB = g.KD / VEC;             // d-blocks per row of the packed side
  const int NBW = kTh / DB;              // n-blocks per workgroup
  const int t = blockIdx.x / tiles_per_slab;
  const int tile = blockIdx.x - t * tiles_per_slab;
  const int db = threadIdx.x % DB;
  const int nb = tile * NBW + threadIdx.x / DB;
  if (nb * VEC >= g.N) return;

  int64_t nchw_off, rows_off;
  slab_offsets(g, t, nchw_off, rows_off);
  // Element offsets of this thread's block on each side.
  const int64_t nchw_base = nchw_off + static_cast<int64_t>(db) * VEC * g.N + nb * VEC;
  const int64_t rows_base = rows_off + static_cast<int64_t>(nb) * VEC * g.KD + db * VEC;
  const char* src = static_cast<const char*>(src_v);
  char* dst = static_cast<char*>(dst_v);
  // Row r of the block on the source side, column c on the destination side.
  const int64_t src_base = kToRows ? nchw_base : rows_base;
  const int64_t src_stride = kToRows ? g.N : g.KD;
  const int64_t dst_base = kToRows ? rows_base : nchw_base;
  const int64_t dst_stride = kToRows ? g.KD : g.N;

  u32x4 in[VEC], out[VEC];
#pragma unroll
  for (int r = 0; r < VEC; ++r) {
    const u32x4* p = reinterpret_cast<const u32x4*>(src + (src_base + r * src_stride) * kEltBytes);
    in[r] = kToRows ? ldg_nt(p) : *p;   // non-temporal reads: measured faster for pack only
  }
  transpose_block(in, out);
#pragma unroll
  for (int c = 0; c < VEC; ++c)
    stg_nt(reinterpret_cast<u32x4*>(dst + (dst_base + c * dst_stride) * kEltBytes), out[c]);
}

// Any N: one thread per element, consecutive threads walk the packed side.
template <typename T, bool kToRows>
__global__ __launch_bounds__(kThreads) void transpose_slabs_scalar(const T* __restrict__ src,
                                                                   T* __restrict__ dst, SlabGeom g,
                                                                   int tiles_per_slab) {
  const int t = blockIdx.x / tiles_per_slab;
  const int tile = blockIdx.x - t * tiles_per_slab;
  const int64_t e = static_cast<int64_t>(tile) * kThreads + threadIdx.x;  // n*KD + d
  if (e >= static_cast<int64_t>(g.N) * g.KD) return;
  const int n = static_cast<int>(e / g.KD);
  const int d = static_cast<int>(e - static_cast<int64_t>(n) * g.KD);
  int64_t nchw_off, rows_off;
  slab_offsets(g, t, nchw_off, rows_off);
  const int64_t nchw_i = nchw_off + static_cast<int64_t>(d) * g.N + n;
  const int64_t rows_i = rows_off + e;
  if (kToRows)
    dst[rows_i] = src[nchw_i];
  else
    dst[nchw_i] = src[rows_i];
}

template <bool kToRows>
hipError_t launch_transpose(const void* src, void* dst, SlabGeom g, int elt_bytes,
                            hipStream_t stream) {
  const int n_slabs = g.BH * g.slots;
  const int vec = 16 / elt_bytes;
  if (g.N % vec == 0) {
    constexpr int th = kToRows ? kThreadsToRows : kThreadsToNchw;
    const int nbw = th / (g.KD / vec);
    const int tiles = (g.N / vec + nbw - 1) / nbw;
    const dim3 grid(static_cast<unsigned>(n_slabs) * tiles);
    if (elt_bytes == 2)
      transpose_slabs_vec<2, kToRows><<<grid, th, 0, stream>>>(src, dst, g, tiles);
    else
      transpose_slabs_vec<4, kToRows><<<grid, th, 0, stream>>>(src, dst, g, tiles);
  } else {
    const int64_t per_slab = static_cast<int64_t>(g.N) * g.KD;
    const int tiles = static_cast<int>((per_slab + kThreads - 1) / kThreads);
    const dim3 grid(static_cast<unsigned>(n_slabs) * tiles);
    if (elt_bytes == 2)
      transpose_slabs_scalar<uint16_t, kToRows><<<grid, kThreads, 0, stream>>>(
          static_cast<const uint16_t*>(src), static_cast<uint16_t*>(dst), g, tiles);
    else
      transpose_slabs_scalar<uint32_t, kToRows><<<grid, kThreads, 0, stream>>>(
          static_cast<const uint32_t*>(src), static_cast<uint32_t*>(dst), g, tiles);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pack_qkv(const void* qkv, void* packed, int BH, int KD, int N, int elt_bytes,
                           hipStream_t stream) {
  return launch_transpose<true>(qkv, packed, SlabGeom{BH, KD, N, 4, 0}, elt_bytes, stream);
}

hipError_t launch_rows_to_nchw(const void* rows, void* nchw, int BH, int KD, int N, int slot0,
                               int elt_bytes, hipStream_t stream) {
  return launch_transpose<false>(rows, nchw, SlabGeom{BH, KD, N, 2, slot0}, elt_bytes, stream);
}

}  // namespace psa
