// CIoU loss, forward and backward, per anchor.
//
// vision-rs book, "Custom Kernels", section "Loss kernels", ciou: predicted and
// target boxes as [4, N] rows (cx, cy, w, h), a per-anchor loss out, and the
// iou, v and alpha the backward reuses instead of recomputing them; one
// workgroup per anchor tile.
//
// The loss is complete-IoU (Zheng et al., AAAI 2020):
//   loss = 1 - IoU + rho^2 / c^2 + alpha * v,
//   v = 4/pi^2 (atan(w_t / h_t) - atan(w_p / h_p))^2, alpha = v / (1 - IoU + v),
// with rho the distance of the two centres and c the diagonal of the smallest
// box enclosing both. eps = 1e-7 guards the divisions (union + eps, c^2 + eps,
// h + eps in the arctangents, alpha's denominator + eps).
//
// The backward gives d(sum dloss * loss)/d(pred) with alpha held constant. It
// reuses the saved iou (dIoU = (dI - IoU dU) / U) and the saved v: since atan
// is increasing, atan(w_t/h_t) - atan(w_p/h_p) has the sign of
// w_t/h_t - w_p/h_p and the magnitude sqrt(v pi^2 / 4), so no arctangent is
// evaluated again.
//
// Both kernels stream: forward 32 bytes in and 16 out per anchor, backward 48
// in and 16 out. Each lane owns four consecutive anchors and moves each row as
// one 16-byte vector when N % 4 == 0; otherwise one anchor per lane.
#include <hip/hip_runtime.h>

#include "psa_device.hpp"
#include "psa_launch.hpp"

namespace psa {
namespace {

constexpr int kThreads = 128;
constexpr float kEps = 1e-7f;
constexpr float kFourOverPi2 = 0.405284734569351086f;  // 4 / pi^2
constexpr float kPi2Over4 = 2.46740110027233966f;      // pi^2 / 4

struct Box {
  float cx, cy, w, h;
};

__device__ __forceinline__ void ciou_fwd_one(Box p, Box g, float& loss, float& iou, float& v,
                                             float& alpha) {
  const float px1 = p.cx - p.w * 0.5f, px2 = p.cx + p.w * 0.5f;
  const float py1 = p.cy - p.h * 0.5f, py2 = p.cy + p.h * 0.5f;
  const float gx1 = g.cx - g.w * 0.5f, gx2 = g.cx + g.w * 0.5f;
  const float gy1 = g.cy - g.h * 0.5f, gy2 = g.cy + g.h * 0.5f;
  const float iw = fmaxf(fminf(px2, gx2) - fmaxf(px1, gx1), 0.0f);
  const float ih = fmaxf(fminf(py2, gy2) - fmaxf(py1, gy1), 0.0f);
  const float inter = iw * ih;
  const float uni = p.w * p.h + g.w * g.h - inter + kEps;
  iou = inter / uni;
  const float cw = fmaxf(px2, gx2) - fminf(px1, gx1);
  const float ch = fmaxf(py2, gy2) - fminf(py1, gy1);
  const float c2 = cw * cw + ch * ch + kEps;
  const float dx = p.cx - g.cx, dy = p.cy - g.cy;
  const float rho2 = dx * dx + dy * dy;
  const float diff = atanf(g.w / (g.h + kEps)) - atanf(p.w / (p.h + kEps));
  v = kFourOverPi2 * diff * diff;
  alpha = v / (v - iou + 1.0f + kEps);
  loss = 1.0f - (iou - rho2 / c2 - alpha * v);
}

// Gradient of dl * loss with respect to (cx, cy, w, h) of the predicted box.
__device__ __forceinline__ Box ciou_bwd_one(Box p, Box g, float iou, float v, float alpha,
                                            float dl) {
  const float px1 = p.cx - p.w * 0.5f, px2 = p.cx + p.w * 0.5f;
  const float py1 = p.cy - p.h * 0.5f, py2 = p.cy + p.h * 0.5f;
  const float gx1 = g.cx - g.w * 0.5f, gx2 = g.cx + g.w * 0.5f;
  const float gy1 = g.cy - g.h * 0.5f, gy2 = g.cy + g.h * 0.5f;
  // Intersection I = iw * ih, union U = w h + w_t h_t - I + eps, IoU = I / U.
  const float iw_raw = fminf(px2, gx2) - fmaxf(px1, gx1);
  const float ih_raw = fminf(py2, gy2) - fmaxf(py1, gy1);
  const float iw = fmaxf(iw_raw, 0.0f), ih = fmaxf(ih_raw, 0.0f);
  const float inter = iw * ih;
  const float uni = p.w * p.h + g.w * g.h - inter + kEps;
  // dI / d(x1, x2, y1, y2): an edge moves the overlap only while it is the inner one.
  const float dI_x1 = (iw_raw > 0.0f && px1 > gx1) ? -ih : 0.0f;
  const float dI_x2 = (iw_raw > 0.0f && px2 < gx2) ? ih : 0.0f;
  const float dI_y1 = (ih_raw > 0.0f && py1 > gy1) ? -iw : 0.0f;
  const float dI_y2 = (ih_raw > 0.0f && py2 < gy2) ? iw : 0.0f;
  // Corners to centre/size: x1 = cx - w/2, x2 = cx + w/2.
  const float dI_cx = dI_x1 + dI_x2, dI_w = 0.5f * (dI_x2 - dI_x1);
  const float dI_cy = dI_y1 + dI_y2, dI_h = 0.5f * (dI_y2 - dI_y1);
  const float inv_u = 1.0f / uni;
  // dIoU = (dI - IoU dU) / U with dU = d(w h) - dI.
  const float diou_cx = (dI_cx + iou * dI_cx) * inv_u;
  const float diou_cy = (dI_cy + iou * dI_cy) * inv_u;
  const float diou_w = (dI_w - iou * (p.h - dI_w)) * inv_u;
  const float diou_h = (dI_h - iou * (p.w - dI_h)) * inv_u;
  // rho^2 / c^2: rho^2 depends on the centre, c^2 on the outer edges.
  const float ex1 = fminf(px1, gx1), ex2 = fmaxf(px2, gx2);
  const float ey1 = fminf(py1, gy1), ey2 = fmaxf(py2, gy2);
  const float cw = ex2 - ex1, ch = ey2 - ey1;
  const float c2 = cw * cw + ch * ch + kEps;
  const float dx = p.cx - g.cx, dy = p.cy - g.cy;
  const float rho2 = dx * dx + dy * dy;
  const float dcw_x1 = px1 < gx1 ? -1.0f : 0.0f, dcw_x2 = px2 > gx2 ? 1.0f : 0.0f;
  const float dch_y1 = py1 < gy1 ? -1.0f : 0.0f, dch_y2 = py2 > gy2 ? 1.0f : 0.0f;
  const float dc2_cx = 2.0f * cw * (dcw_x1 + dcw_x2), dc2_w = cw * (dcw_x2 - dcw_x1);
  const float dc2_cy = 2.0f * ch * (dch_y1 + dch_y2), dc2_h = ch * (dch_y2 - dch_y1);
  const float inv_c2 = 1.0f / c2, ratio = rho2 * inv_c2;
  const float dr_cx = (2.0f * dx - ratio * dc2_cx) * inv_c2;
  const float dr_cy = (2.0f * dy - ratio * dc2_cy) * inv_c2;
  const float dr_w = -ratio * dc2_w * inv_c2;
  const float dr_h = -ratio * dc2_h * inv_c2;
  // v = k diff^2, diff = atan(w_t/(h_t+eps)) - atan(w/(h+eps)); |diff| from the saved v.
  const float he = p.h + kEps;
  const float rt = g.w / (g.h + kEps), rp = p.w / he;
  const float mag = sqrtf(v * kPi2Over4);
  const float diff = rt > rp ? mag : (rt < rp ? -mag : 0.0f);
  const float q = -2.0f * kFourOverPi2 * diff / (he * he + p.w * p.w);
  const float dv_w = q * he, dv_h = -q * p.w;
  Box d;
  d.cx = dl * (dr_cx - diou_cx);
  d.cy = dl * (dr_cy - diou_cy);
  d.w = dl * (dr_w - diou_w + alpha * dv_w);
  d.h = dl * (dr_h - diou_h + alpha * dv_h);
  return d;
}

typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ Box box_at(const f4* r, int k) {
  return Box{r[0][k], r[1][k], r[2][k], r[3][k]};
}

// Vector path (N % 4 == 0): rows are [4, N] with each row 16-byte aligned.
__global__ __launch_bounds__(kThreads) void ciou_fwd_vec(const float* __restrict__ pred,
                                                         const float* __restrict__ target,
                                                         float* __restrict__ loss,
                                                         float* __restrict__ iou,
                                                         float* __restrict__ v,
                                                         float* __restrict__ alpha, int64_t N) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i * 4 >= N) return;
  const int64_t N4 = N / 4;
  const f4* P = reinterpret_cast<const f4*>(pred);
  const f4* G = reinterpret_cast<const f4*>(target);
  f4 p[4], g[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    p[c] = ldg_nt(P + c * N4 + i);
    g[c] = ldg_nt(G + c * N4 + i);
  }
  __builtin_amdgcn_sched_barrier(0);   // all eight loads ahead of the arithmetic
  f4 lo, io, vo, ao;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float l, u, vv, a;
    ciou_fwd_one(box_at(p, k), box_at(g, k), l, u, vv, a);
    lo[k] = l;
    io[k] = u;
    vo[k] = vv;
    ao[k] = a;
  }
  stg_nt(reinterpret_cast<f4*>(loss) + i, lo);
  stg_nt(reinterpret_cast<f4*>(iou) + i, io);
  stg_nt(reinterpret_cast<f4*>(v) + i, vo);
  stg_nt(reinterpret_cast<f4*>(alpha) + i, ao);
}

__global__ __launch_bounds__(kThreads) void ciou_fwd_scalar(const float* __restrict__ pred,
                                                            const float* __restrict__ target,
                                                            float* __restrict__ loss,
                                                            float* __restrict__ iou,
                                                            float* __restrict__ v,
                                                            float* __restrict__ alpha, int64_t N) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= N) return;
  const Box p{ldg_nt(pred + i), ldg_nt(pred + N + i), ldg_nt(pred + 2 * N + i),
              ldg_nt(pred + 3 * N + i)};
  const Box g{ldg_nt(target + i), ldg_nt(target + N + i), ldg_nt(target + 2 * N + i),
              ldg_nt(target + 3 * N + i)};
  float l, u, vv, a;
  ciou_fwd_one(p, g, l, u, vv, a);
  stg_nt(loss + i, l);
  stg_nt(iou + i, u);
  stg_nt(v + i, vv);
  stg_nt(alpha + i, a);
}

__global__ __launch_bounds__(kThreads) void ciou_bwd_vec(
    const float* __restrict__ pred, const float* __restrict__ target, const float* __restrict__ iou,
    const float* __restrict__ v, const float* __restrict__ alpha, const float* __restrict__ dloss,
    float* __restrict__ dpred, int64_t N) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i * 4 >= N) return;
  const int64_t N4 = N / 4;
  const f4* P = reinterpret_cast<const f4*>(pred);
  const f4* G = reinterpret_cast<const f4*>(target);
  f4 p[4], g[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    p[c] = ldg_nt(P + c * N4 + i);
    g[c] = ldg_nt(G + c * N4 + i);
  }
  const f4 u = ldg_nt(reinterpret_cast<const f4*>(iou) + i);
  const f4 vv = ldg_nt(reinterpret_cast<const f4*>(v) + i);
  const f4 a = ldg_nt(reinterpret_cast<const f4*>(alpha) + i);
  const f4 dl = ldg_nt(reinterpret_cast<const f4*>(dloss) + i);
  // Keep all twelve loads ahead of the arithmetic (the scheduler would otherwise
  // sink some of them to their first use, each then waited for on its own).
  __builtin_amdgcn_sched_barrier(0);
  f4 o[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const Box d = ciou_bwd_one(box_at(p, k), box_at(g, k), u[k], vv[k], a[k], dl[k]);
    o[0][k] = d.cx;
    o[1][k] = d.cy;
    o[2][k] = d.w;
    o[3][k] = d.h;
  }
  f4* D = reinterpret_cast<f4*>(dpred);
#pragma unroll
  for (int c = 0; c < 4; ++c) stg_nt(D + c * N4 + i, o[c]);
}

__global__ __launch_bounds__(kThreads) void ciou_bwd_scalar(
    const float* __restrict__ pred, const float* __restrict__ target, const float* __restrict__ iou,
    const float* __restrict__ v, const float* __restrict__ alpha, const float* __restrict__ dloss,
    float* __restrict__ dpred, int64_t N) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= N) return;
  const Box p{ldg_nt(pred + i), ldg_nt(pred + N + i), ldg_nt(pred + 2 * N + i),
              ldg_nt(pred + 3 * N + i)};
  const Box g{ldg_nt(target + i), ldg_nt(target + N + i), ldg_nt(target + 2 * N + i),
              ldg_nt(target + 3 * N + i)};
  const Box d = ciou_bwd_one(p, g, ldg_nt(iou + i), ldg_nt(v + i), ldg_nt(alpha + i),
                             ldg_nt(dloss + i));
  stg_nt(dpred + i, d.cx);
  stg_nt(dpred + N + i, d.cy);
  stg_nt(dpred + 2 * N + i, d.w);
  stg_nt(dpred + 3 * N + i, d.h);
}

unsigned grid_for(int64_t lanes) { return static_cast<unsigned>((lanes + kThreads - 1) / kThreads); }

}  // namespace

hipError_t launch_ciou_fwd(const float* pred, const float* target, float* loss, float* iou,
                           float* v, float* alpha, int64_t N, hipStream_t stream) {
  if (N % 4 == 0)
    hipLaunchKernelGGL(ciou_fwd_vec, dim3(grid_for(N / 4)), dim3(kThreads), 0, stream, pred,
                       target, loss, iou, v, alpha, N);
  else
    hipLaunchKernelGGL(ciou_fwd_scalar, dim3(grid_for(N)), dim3(kThreads), 0, stream, pred,
                       target, loss, iou, v, alpha, N);
  return hipGetLastError();
}

hipError_t launch_ciou_bwd(const float* pred, const float* target, const float* iou,
                           const float* v, const float* alpha, const float* dloss, float* dpred,
                           int64_t N, hipStream_t stream) {
  if (N % 4 == 0)
    hipLaunchKernelGGL(ciou_bwd_vec, dim3(grid_for(N / 4)), dim3(kThreads), 0, stream, pred,
                       target, iou, v, alpha, dloss, dpred, N);
  else
    hipLaunchKernelGGL(ciou_bwd_scalar, dim3(grid_for(N)), dim3(kThreads), 0, stream, pred,
                       target, iou, v, alpha, dloss, dpred, N);
  return hipGetLastError();
}

}  // namespace psa
