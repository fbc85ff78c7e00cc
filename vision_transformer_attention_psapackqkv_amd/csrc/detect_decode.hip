// Detect-decode: raw LTRB box distances + a per-anchor grid -> [cx, cy, w, h].
//
// vision-rs book, "Custom Kernels", section "Detect-decode": one fused pass over
// the model's box predictions and a precomputed anchor grid (anchor_x,
// anchor_y, strides). The teenygrad book, "Your Kernel as a Graph Op", section
// "A real one": boxes are [B, 4, A] and the op keeps that shape.
//
// Per anchor a of batch item b (distances and anchor in grid units, result in
// pixels): x1 = ax - l, y1 = ay - t, x2 = ax + r, y2 = ay + b, then
// cx = (x1 + x2)/2 * s, cy = (y1 + y2)/2 * s, w = (x2 - x1) * s, h = (y2 - y1) * s.
//
// The op is a stream: 4 loads and 4 stores per anchor and batch item, the
// anchor grid (12 bytes per anchor) read by every batch item and kept in L2.
// Each lane owns VEC consecutive anchors of one batch row and moves them as
// 16-byte vectors per channel; box data are streamed with non-temporal loads
// and stores so they do not push the anchor grid out of the caches.
#include <hip/hip_runtime.h>

#include "psa_device.hpp"
#include "psa_launch.hpp"

namespace psa {
namespace {

constexpr int kThreads = 128;

template <typename T>
struct Elt;
template <>
struct Elt<float> {
  __device__ static float get(float x) { return x; }
  __device__ static float put(float x) { return x; }
};
template <>
struct Elt<uint16_t> {
  __device__ static float get(uint16_t x) { return bf16_bits_to_float(x); }
  __device__ static uint16_t put(float x) { return float_to_bf16_bits(x); }
};

__device__ __forceinline__ void decode_one(float l, float t, float r, float b, float ax, float ay,
                                           float s, float& cx, float& cy, float& w, float& h) {
  const float x1 = ax - l, y1 = ay - t, x2 = ax + r, y2 = ay + b;
  cx = (x1 + x2) * 0.5f * s;
  cy = (y1 + y2) * 0.5f * s;
  w = (x2 - x1) * s;
  h = (y2 - y1) * s;
}

// Vector path: A % VEC == 0, so every channel row of every batch item starts on
// a 16-byte boundary. blockIdx.y is the batch item, blockIdx.x a tile of
// kThreads * VEC anchors.
template <typename T, int VEC>
__global__ __launch_bounds__(kThreads) void detect_decode_vec(const T* __restrict__ boxes,
                                                              const float* __restrict__ anchor_x,
                                                              const float* __restrict__ anchor_y,
                                                              const float* __restrict__ strides,
                                                              T* __restrict__ out, int64_t A) {
  static_assert(VEC * sizeof(T) == 16, "one 16-byte vector per channel");
  typedef T TV __attribute__((ext_vector_type(VEC)));
  typedef float FV __attribute__((ext_vector_type(4)));
  const int64_t a0 = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) * VEC;
  if (a0 >= A) return;
  const int64_t row = static_cast<int64_t>(blockIdx.y) * 4 * A;
  TV d[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) d[c] = ldg_nt(reinterpret_cast<const TV*>(boxes + row + c * A + a0));
  float ax[VEC], ay[VEC], st[VEC];
#pragma unroll
  for (int k = 0; k < VEC; k += 4) {
    const FV x = *reinterpret_cast<const FV*>(anchor_x + a0 + k);
    const FV y = *reinterpret_cast<const FV*>(anchor_y + a0 + k);
    const FV s = *reinterpret_cast<const FV*>(strides + a0 + k);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ax[k + j] = x[j];
      ay[k + j] = y[j];
      st[k + j] = s[j];
    }
  }
  TV o[4];
#pragma unroll
  for (int k = 0; k < VEC; ++k) {
    float cx, cy, w, h;
    decode_one(Elt<T>::get(d[0][k]), Elt<T>::get(d[1][k]), Elt<T>::get(d[2][k]),
               Elt<T>::get(d[3][k]), ax[k], ay[k], st[k], cx, cy, w, h);
    o[0][k] = Elt<T>::put(cx);
    o[1][k] = Elt<T>::put(cy);
    o[2][k] = Elt<T>::put(w);
    o[3][k] = Elt<T>::put(h);
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) stg_nt(reinterpret_cast<TV*>(out + row + c * A + a0), o[c]);
}

// Any A: one anchor per lane (each wave still reads 64 consecutive elements per channel).
template <typename T>
__global__ __launch_bounds__(kThreads) void detect_decode_scalar(const T* __restrict__ boxes,
                                                                 const float* __restrict__ anchor_x,
                                                                 const float* __restrict__ anchor_y,
                                                                 const float* __restrict__ strides,
                                                                 T* __restrict__ out, int64_t A) {
  const int64_t a = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (a >= A) return;
  const int64_t row = static_cast<int64_t>(blockIdx.y) * 4 * A;
  float d[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) d[c] = Elt<T>::get(ldg_nt(boxes + row + c * A + a));
  float cx, cy, w, h;
  decode_one(d[0], d[1], d[2], d[3], anchor_x[a], anchor_y[a], strides[a], cx, cy, w, h);
  stg_nt(out + row + 0 * A + a, Elt<T>::put(cx));
  stg_nt(out + row + 1 * A + a, Elt<T>::put(cy));
  stg_nt(out + row + 2 * A + a, Elt<T>::put(w));
  stg_nt(out + row + 3 * A + a, Elt<T>::put(h));
}

template <typename T>
hipError_t launch_typed(const void* boxes, const float* ax, const float* ay, const float* st,
                        void* out, int B, int64_t A, hipStream_t stream) {
  constexpr int VEC = 16 / sizeof(T);
  const T* in = static_cast<const T*>(boxes);
  T* o = static_cast<T*>(out);
  if (A % VEC == 0) {
    const int64_t tiles = (A / VEC + kThreads - 1) / kThreads;
    hipLaunchKernelGGL((detect_decode_vec<T, VEC>), dim3(static_cast<unsigned>(tiles), B),
                       dim3(kThreads), 0, stream, in, ax, ay, st, o, A);
  } else {
    const int64_t tiles = (A + kThreads - 1) / kThreads;
    hipLaunchKernelGGL((detect_decode_scalar<T>), dim3(static_cast<unsigned>(tiles), B),
                       dim3(kThreads), 0, stream, in, ax, ay, st, o, A);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_detect_decode(const void* boxes, const float* anchor_x, const float* anchor_y,
                                const float* strides, void* out, int B, int64_t A, bool bf16,
                                hipStream_t stream) {
  return bf16 ? launch_typed<uint16_t>(boxes, anchor_x, anchor_y, strides, out, B, A, stream)
              : launch_typed<float>(boxes, anchor_x, anchor_y, strides, out, B, A, stream);
}

}  // namespace psa
