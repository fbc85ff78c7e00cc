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
// A workgroup (256 threads for pack, 512 for merge and extract) moves one
// tile of a slab (all KD channels x tile_bytes / (KD * elt) pixels) through LDS:
// 16-byte loads along the side the data is contiguous on, the transpose
// between LDS and registers, 16-byte stores along the other side, so that
// every wave instruction reads or writes 1 KB of contiguous runs
// on both sides (whole channel-row runs on the NCHW side, whole consecutive
// rows on the packed side). Rows whose start is not 16-byte aligned (N not a
// multiple of 16 bytes / element size), and slabs of 2 GB or more, take a
// scalar kernel instead. Measured
// on MI355X at the 80x80 map, this beats an 8x8-block register transpose (whose
// wave instructions touch 8 separate 128-byte runs) by 4-7 % and torch's device
// copy of pack's bytes by ~11 %.
#include <type_traits>

#include "psa_device.hpp"
#include "psa_launch.hpp"

namespace psa {
namespace {

constexpr int kThreads = 256;   // scalar kernel

// Cache-policy operand of a gfx950 buffer store: sc0 (1) | nt (2) | sc1 (16).
constexpr int kStoreScNtSc = 1 | 2 | 16;

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

// One tile = all KD channels x PX pixels of one slab (tile_bytes of data), staged in
// LDS so that both global sides move in long contiguous runs: 16-byte chunk q
// of the NCHW side is (row q / CPR, column q % CPR), so one wave instruction
// covers 1 KB of whole channel-row runs; chunk q of the packed side is (pixel
// q / (KD / VEC), channel block q % (KD / VEC)), so one wave instruction covers
// whole consecutive packed rows (1 KB contiguous at KD = 64). The transpose
// happens between LDS and registers, one element at a time on the side the
// chunk does not run along. LDS chunk columns are XOR-swizzled by the row's
// channel block, so the 8 rows (4 for f32) one packed-side chunk gathers from
// sit in different bank groups.
// Tile bytes and workgroup size, measured best for each direction on MI355X at
// the 80x80 map: pack moves 16 KB tiles with 256 threads (4 chunks per
// thread); merge and extract move 8 KB tiles with 512 threads (one chunk per
// thread; 16 KB at key_dim 128, whose 8 KB tile would have fewer than 8
// chunks per channel row), which with their sc0 nt sc1 stores measured 1.5-2 %
// faster than 16 KB tiles.
template <bool kToRows, int KD>
constexpr int tile_bytes() { return kToRows || KD >= 128 ? 16384 : 8192; }
template <bool kToRows>
constexpr int threads_lds() { return kToRows ? 256 : 512; }

template <int kElt>
struct Word;
template <>
struct Word<2> { using T = uint16_t; };
template <>
struct Word<4> { using T = uint32_t; };

// kToRows = true: NCHW [KD, N] slabs -> packed [N, KD] slabs (pack).
// kToRows = false: packed [N, KD] slabs -> NCHW [KD, N] slabs (merge, extract).
// Workgroup i of a launch moves tile i % tiles_per_slab of slab slab0 + i / tiles_per_slab.
template <int kElt, int KD, bool kToRows, int kThreadsLds = threads_lds<kToRows>()>
__global__ __launch_bounds__(kThreadsLds) void transpose_slabs_lds(const void* __restrict__ src_v,
                                                                   void* __restrict__ dst_v,
                                                                   SlabGeom g, int tiles_per_slab,
                                                                   int slab0) {
  using T = typename Word<kElt>::T;
  constexpr int VEC = 16 / kElt;                 // elements per 16-byte chunk
  constexpr int PX = tile_bytes<kToRows, KD>() / (KD * kElt);   // pixels per tile
  constexpr int CPR = PX / VEC;                  // chunks per channel row of a tile (>= 8)
  constexpr int DBN = KD / VEC;                  // chunks per packed row
  constexpr int PER = KD * CPR / kThreadsLds;    // chunks per thread
  static_assert(CPR >= 8 && (CPR & (CPR - 1)) == 0 && KD * CPR == PER * kThreadsLds, "tile shape");
  __shared__ __attribute__((aligned(16))) T lds[KD * PX];

  const int local = blockIdx.x / tiles_per_slab;
  const int tile = blockIdx.x - local * tiles_per_slab;
  const int t = slab0 + local;
  const int p0 = tile * PX;
  const int np = min(PX, g.N - p0);   // pixels of this tile; a multiple of VEC
  int64_t nchw_off, rows_off;
  slab_offsets(g, t, nchw_off, rows_off);
  const T* src = static_cast<const T*>(src_v);
  T* dst = static_cast<T*>(dst_v);
  // LDS element index of (channel row, pixel) inside the tile.
  auto at = [](int row, int px) { return row * PX + (((px / VEC) ^ ((row / VEC) & 7)) * VEC) + px % VEC; };

  // Only the global stores are guarded. Loads past the tile's last pixel (the
  // short last tile of a slab) are clamped to its last chunk, so every load is
  // unconditional and all of a thread's loads are in flight together (a load
  // under a branch would be waited for inside that branch); LDS positions past
  // it hold those duplicates and are never stored.
  u32x4 v[PER];
  if constexpr (kToRows) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int q = u * kThreadsLds + threadIdx.x, row = q / CPR, col = q % CPR;
      const int p = min(col * VEC, np - VEC);
      v[u] = ldg_nt(reinterpret_cast<const u32x4*>(src + nchw_off + static_cast<int64_t>(row) * g.N + p0 + p));
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int q = u * kThreadsLds + threadIdx.x, row = q / CPR, col = q % CPR;
      *reinterpret_cast<u32x4*>(&lds[at(row, col * VEC)]) = v[u];
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int q = u * kThreadsLds + threadIdx.x, px = q / DBN, cb = q % DBN;
      u32x4 w;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if constexpr (kElt == 2)
          w[k] = uint32_t(lds[at(cb * VEC + 2 * k, px)]) | (uint32_t(lds[at(cb * VEC + 2 * k + 1, px)]) << 16);
        else
          w[k] = lds[at(cb * VEC + k, px)];
      }
      if (px < np)
        stg_nt(reinterpret_cast<u32x4*>(dst + rows_off + static_cast<int64_t>(p0 + px) * KD + cb * VEC), w);
    }
  } else {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int q = u * kThreadsLds + threadIdx.x, px = q / DBN, cb = q % DBN;
      const int p = min(px, np - 1);
      v[u] = ldg_nt(reinterpret_cast<const u32x4*>(src + rows_off + static_cast<int64_t>(p0 + p) * KD + cb * VEC));
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int q = u * kThreadsLds + threadIdx.x, px = q / DBN, cb = q % DBN;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if constexpr (kElt == 2) {
          lds[at(cb * VEC + 2 * k, px)] = static_cast<T>(v[u][k] & 0xFFFFu);
          lds[at(cb * VEC + 2 * k + 1, px)] = static_cast<T>(v[u][k] >> 16);
        } else {
          lds[at(cb * VEC + k, px)] = v[u][k];
        }
      }
    }
    __syncthreads();
    // NCHW-side stores as buffer stores over the slab (under 2 GB: the
    // launcher checks) with the non-temporal and both scope bits set (sc0 nt
    // sc1): measured 1-1.5 % faster than plain non-temporal stores at the
    // 80x80 map (with 16 KB tiles), while the same bits on the loads, or on
    // pack's stores, were not faster.
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(dst + nchw_off, 0, KD * g.N * kElt, kBufferWord3);
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int q = u * kThreadsLds + threadIdx.x, row = q / CPR, col = q % CPR;
      const u32x4 w = *reinterpret_cast<const u32x4*>(&lds[at(row, col * VEC)]);
      if (col * VEC < np)
        __builtin_amdgcn_raw_buffer_store_b128(w, rs, (row * g.N + p0 + col * VEC) * kElt, 0, kStoreScNtSc);
    }
  }
}

// Any N: one thread per element, consecutive threads walk the packed side. The grid
// is capped (a launch holds fewer than 2^32 work-items) and strides over the
// n_slabs * tiles_per_slab tiles of kThreads elements.
template <typename T, bool kToRows>
__global__ __launch_bounds__(kThreads) void transpose_slabs_scalar(const T* __restrict__ src,
                                                                   T* __restrict__ dst, SlabGeom g,
                                                                   int64_t tiles_per_slab, int64_t tiles) {
  const int64_t per_slab = static_cast<int64_t>(g.N) * g.KD;
  for (int64_t i = blockIdx.x; i < tiles; i += gridDim.x) {
    const int t = static_cast<int>(i / tiles_per_slab);
    const int64_t e = (i - t * tiles_per_slab) * kThreads + threadIdx.x;  // n*KD + d
    if (e >= per_slab) continue;
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
}

// Workgroups per launch: a launch holds fewer than 2^32 work-items; 2^31 keeps a margin.
constexpr int64_t kMaxLaunchItems = int64_t(1) << 31;

template <int kElt, bool kToRows>
void launch_lds(const void* src, void* dst, SlabGeom g, int n_slabs, hipStream_t stream) {
  auto go = [&](auto kd) {
    constexpr int KD = decltype(kd)::value;
    constexpr int PX = tile_bytes<kToRows, KD>() / (KD * kElt);
    const int tiles = (g.N + PX - 1) / PX;
    // Whole slabs per launch, as many as one launch holds: pack takes a single launch up to
    // 128 GB of slabs, merge and extract up to 32 GB, larger calls several.
    const int64_t per_launch = kMaxLaunchItems / (static_cast<int64_t>(tiles) * threads_lds<kToRows>());
    for (int64_t s0 = 0; s0 < n_slabs; s0 += per_launch) {
      const int64_t n = n_slabs - s0 < per_launch ? n_slabs - s0 : per_launch;
      const dim3 grid(static_cast<unsigned>(n * tiles));
      transpose_slabs_lds<kElt, KD, kToRows><<<grid, threads_lds<kToRows>(), 0, stream>>>(
          src, dst, g, tiles, static_cast<int>(s0));
    }
  };
  switch (g.KD) {
    case 16: go(std::integral_constant<int, 16>{}); break;
    case 32: go(std::integral_constant<int, 32>{}); break;
    case 64: go(std::integral_constant<int, 64>{}); break;
    default: go(std::integral_constant<int, 128>{}); break;
  }
}

template <bool kToRows>
hipError_t launch_transpose(const void* src, void* dst, SlabGeom g, int elt_bytes,
                            hipStream_t stream) {
  const int n_slabs = g.BH * g.slots;
  const int vec = 16 / elt_bytes;
  if (g.KD != 16 && g.KD != 32 && g.KD != 64 && g.KD != 128) return hipErrorInvalidValue;
  // The LDS kernel needs 16-byte aligned rows and, for its buffer stores, slabs
  // under 2 GB; anything else takes the scalar kernel.
  if (g.N % vec == 0 && static_cast<int64_t>(g.N) * g.KD * elt_bytes < (int64_t(1) << 31)) {
    if (elt_bytes == 2)
      launch_lds<2, kToRows>(src, dst, g, n_slabs, stream);
    else
      launch_lds<4, kToRows>(src, dst, g, n_slabs, stream);
  } else {
    const int64_t per_slab = static_cast<int64_t>(g.N) * g.KD;
    const int64_t tiles_per_slab = (per_slab + kThreads - 1) / kThreads;
    const int64_t tiles = tiles_per_slab * n_slabs;
    const int64_t cap = kMaxLaunchItems / kThreads;
    const dim3 grid(static_cast<unsigned>(tiles < cap ? tiles : cap));
    if (elt_bytes == 2)
      transpose_slabs_scalar<uint16_t, kToRows><<<grid, kThreads, 0, stream>>>(
          static_cast<const uint16_t*>(src), static_cast<uint16_t*>(dst), g, tiles_per_slab, tiles);
    else
      transpose_slabs_scalar<uint32_t, kToRows><<<grid, kThreads, 0, stream>>>(
          static_cast<const uint32_t*>(src), static_cast<uint32_t*>(dst), g, tiles_per_slab, tiles);
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
