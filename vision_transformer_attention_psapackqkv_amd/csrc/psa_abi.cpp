// The C ABI of libpsa: argument validation, then one launcher call.
//
// teenygrad's book ("Wiring the Runtime", "Packing arguments") warns that a
// launch-time op description passes pointers and i32 dims in kernel-parameter
// order with nothing checking them. Here every entry point checks every
// argument before anything is enqueued and reports the first failure with the
// entry point's name ("Your Kernel as a Graph Op", "What the lowering does
// with it": errors name the op).
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "../../include/psa.h"
#include "psa_launch.hpp"

static_assert(psa::kNoAllocScratchBytes == PSA_NOALLOC_SCRATCH_BYTES,
              "the scratch array and the limit the header states must agree");

namespace {

thread_local std::string g_last_error;

psa_status fail(psa_status st, const char* fn, const char* fmt, ...) {
  char msg[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(msg, sizeof(msg), fmt, ap);
  va_end(ap);
  g_last_error = std::string(fn) + ": " + msg;
  return st;
}

psa_status ok() {
  g_last_error.clear();
  return PSA_OK;
}

bool supported_dim(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

int elt_bytes(psa_dtype t) { return t == PSA_BF16 ? 2 : 4; }

struct Range {
  const char* name;
  uintptr_t lo, hi;  // [lo, hi)
};

Range range(const char* name, const void* p, int64_t elems, int64_t elt) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{name, lo, lo + static_cast<uintptr_t>(elems * elt)};
}

bool overlap(const Range& a, const Range& b) { return a.lo < b.hi && b.lo < a.hi; }

// Checks a dtype, that dims are positive and that a product stays far below
// int64 and int32 limits used for grids and slab strides.
psa_status check_dtype(const char* fn, psa_dtype dtype) {
  if (dtype != PSA_F32 && dtype != PSA_BF16)
    return fail(PSA_ERR_UNSUPPORTED, fn, "dtype=%d is neither PSA_F32 (0) nor PSA_BF16 (1)",
                static_cast<int>(dtype));
  return PSA_OK;
}

psa_status check_aligned(const char* fn, const char* name, const void* p) {
  if (reinterpret_cast<uintptr_t>(p) % 16 != 0)
    return fail(PSA_ERR_ALIGN, fn, "%s=%p is not 16-byte aligned", name, p);
  return PSA_OK;
}

psa_status check_disjoint(const char* fn, const Range* r, int n) {
  for (int i = 0; i < n; ++i)
    for (int j = i + 1; j < n; ++j)
      if (r[i].lo != 0 && r[j].lo != 0 && overlap(r[i], r[j]))
        return fail(PSA_ERR_ALIAS, fn, "%s and %s overlap", r[i].name, r[j].name);
  return PSA_OK;
}

// r[0, n_in) are inputs, r[n_in, n) outputs: inputs may share memory, but
// every output must be disjoint from every other range.
psa_status check_outputs_disjoint(const char* fn, const Range* r, int n, int n_in) {
  for (int i = n_in; i < n; ++i)
    for (int j = 0; j < n; ++j)
      if (j != i && overlap(r[i], r[j]))
        return fail(PSA_ERR_ALIAS, fn, "%s and %s overlap", r[i].name, r[j].name);
  return PSA_OK;
}

// Largest element count of the one-lane-per-element launches (below 2^31 work-items).
constexpr int64_t kMaxLanes = (int64_t(1) << 31) - 256;

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Runs an entry point's launches. HIP keeps one "last error" per thread, set
// by any earlier failing HIP call and returned (and cleared) by the next
// hipGetLastError(); the launchers report their launches with that call. It is
// cleared first, so that a failure left behind by an unrelated earlier call is
// not reported as this entry point's launch failure. (An error that poisons the
// device stays sticky and is still reported.) Before the launches it runs the
// device set-up, which does its work on the first call on each device only.
template <typename Launch>
psa_status launched(const char* fn, Launch&& launch) {
  (void)hipGetLastError();
  const hipError_t init = psa::init_device();
  if (init != hipSuccess)
    return fail(PSA_ERR_LAUNCH, fn, "device set-up failed: %s", hipGetErrorString(init));
  const hipError_t e = launch();
  if (e != hipSuccess) return fail(PSA_ERR_LAUNCH, fn, "launch failed: %s", hipGetErrorString(e));
  return ok();
}

// Shared checks of the NCHW-side entry points. Element counts go to *n_in / *n_out.
psa_status check_map(const char* fn, int B, int heads, int key_dim, int H, int W,
                     psa_dtype dtype) {
  if (B <= 0 || heads <= 0 || key_dim <= 0 || H <= 0 || W <= 0)
    return fail(PSA_ERR_SHAPE, fn, "dims must be > 0 (B=%d heads=%d key_dim=%d H=%d W=%d)", B,
                heads, key_dim, H, W);
  if (!supported_dim(key_dim))
    return fail(PSA_ERR_UNSUPPORTED, fn, "key_dim=%d is not one of 16, 32, 64, 128", key_dim);
  if (psa_status st = check_dtype(fn, dtype)) return st;
  const int64_t N = static_cast<int64_t>(H) * W;
  const int64_t BH = static_cast<int64_t>(B) * heads;
  // Grids are sized in int32 workgroups and slab strides in int64 elements.
  if (N > (1 << 28) || BH > (1 << 24) || BH * 4 * key_dim * N > (int64_t(1) << 40))
    return fail(PSA_ERR_SHAPE, fn, "sizes too large (BH=%lld N=%lld key_dim=%d)",
                static_cast<long long>(BH), static_cast<long long>(N), key_dim);
  return PSA_OK;
}

// The attention kernels give each 128 rows (queries, or keys for dK/dV) one
// workgroup of up to 256 work-items, and a launch holds fewer than 2^32
// work-items: BH * n rounded up to 128 rows stays below 2^31 - 2^23.
psa_status check_launch_rows(const char* fn, int64_t BH, int64_t n) {
  const int64_t rows = BH * ((n + 127) / 128) * 128;
  if (rows >= (int64_t(1) << 31) - (int64_t(1) << 23))
    return fail(PSA_ERR_SHAPE, fn, "BH=%lld times %lld rows is too many for one launch (at most 2^31 - 2^23)",
                static_cast<long long>(BH), static_cast<long long>(n));
  return PSA_OK;
}

psa_status check_attn(const char* fn, int BH, int n_q, int n_k, int head_dim, float scale,
                      psa_dtype dtype) {
  if (BH <= 0 || n_q <= 0 || n_k <= 0 || head_dim <= 0)
    return fail(PSA_ERR_SHAPE, fn, "dims must be > 0 (BH=%d n_q=%d n_k=%d head_dim=%d)", BH, n_q,
                n_k, head_dim);
  if (!supported_dim(head_dim))
    return fail(PSA_ERR_UNSUPPORTED, fn, "head_dim=%d is not one of 16, 32, 64, 128", head_dim);
  if (psa_status st = check_dtype(fn, dtype)) return st;
  if (!std::isfinite(scale) || !(scale > 0.0f))
    return fail(PSA_ERR_UNSUPPORTED, fn, "scale=%g must be finite and > 0", static_cast<double>(scale));
  const int64_t rows = static_cast<int64_t>(BH) * (n_q > n_k ? n_q : n_k);
  if (n_q > (1 << 28) || n_k > (1 << 28) || rows * head_dim > (int64_t(1) << 40))
    return fail(PSA_ERR_SHAPE, fn, "sizes too large (BH=%d n_q=%d n_k=%d)", BH, n_q, n_k);
  return check_launch_rows(fn, BH, n_q > n_k ? n_q : n_k);
}

#define PSA_TRY(expr)                       \
  do {                                      \
    if (psa_status st_ = (expr)) return st_; \
  } while (0)

psa_status layout_entry(const char* fn, const void* in, void* out, int B, int heads, int key_dim,
                        int H, int W, psa_dtype dtype, int in_slots, int out_slots) {
  if (!in) return fail(PSA_ERR_NULL, fn, "input pointer is NULL");
  if (!out) return fail(PSA_ERR_NULL, fn, "output pointer is NULL");
  PSA_TRY(check_map(fn, B, heads, key_dim, H, W, dtype));
  PSA_TRY(check_aligned(fn, "input", in));
  PSA_TRY(check_aligned(fn, "output", out));
  const int64_t per_slot = static_cast<int64_t>(B) * heads * key_dim * H * W;
  const Range r[2] = {range("input", in, per_slot * in_slots, elt_bytes(dtype)),
                      range("output", out, per_slot * out_slots, elt_bytes(dtype))};
  return check_disjoint(fn, r, 2);
}

}  // namespace

extern "C" {

psa_status psa_pack_qkv(const void* qkv_nchw, void* packed, int B, int heads, int key_dim, int H,
                        int W, psa_dtype dtype, void* stream) {
  const char* fn = "psa_pack_qkv";
  PSA_TRY(layout_entry(fn, qkv_nchw, packed, B, heads, key_dim, H, W, dtype, 4, 4));
  return launched(fn, [&] {
    return psa::launch_pack_qkv(qkv_nchw, packed, B * heads, key_dim, H * W, elt_bytes(dtype),
                                as_stream(stream));
  });
}

psa_status psa_extract_v(const void* packed, void* v_nchw, int B, int heads, int key_dim, int H,
                         int W, psa_dtype dtype, void* stream) {
  const char* fn = "psa_extract_v";
  PSA_TRY(layout_entry(fn, packed, v_nchw, B, heads, key_dim, H, W, dtype, 4, 2));
  return launched(fn, [&] {
    return psa::launch_rows_to_nchw(packed, v_nchw, B * heads, key_dim, H * W, 2, elt_bytes(dtype),
                                    as_stream(stream));
  });
}

psa_status psa_merge_attn(const void* o2, void* out_nchw, int B, int heads, int key_dim, int H,
                          int W, psa_dtype dtype, void* stream) {
  const char* fn = "psa_merge_attn";
  PSA_TRY(layout_entry(fn, o2, out_nchw, B, heads, key_dim, H, W, dtype, 2, 2));
  return launched(fn, [&] {
    return psa::launch_rows_to_nchw(o2, out_nchw, B * heads, key_dim, H * W, 0, elt_bytes(dtype),
                                    as_stream(stream));
  });
}

size_t fa2_fwd_workspace_bytes(int BH, int n_q, int n_k, int head_dim, psa_dtype dtype) {
  if (BH <= 0 || n_q <= 0 || n_k <= 0 || !supported_dim(head_dim) ||
      (dtype != PSA_F32 && dtype != PSA_BF16))
    return 0;
  return psa::fa2_fwd_split_bytes(BH, n_q, n_k, head_dim, dtype == PSA_BF16);
}

psa_status fa2_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int BH,
                   int n_q, int n_k, int head_dim, float scale, psa_dtype dtype, void* workspace,
                   size_t workspace_bytes, void* stream) {
  const char* fn = "fa2_fwd";
  if (!q || !k || !v || !o)
    return fail(PSA_ERR_NULL, fn, "q, k, v and o must not be NULL (lse and workspace may be)");
  PSA_TRY(check_attn(fn, BH, n_q, n_k, head_dim, scale, dtype));
  const char* names[6] = {"q", "k", "v", "o", "lse", "workspace"};
  const void* ptrs[6] = {q, k, v, o, lse, workspace};
  for (int i = 0; i < 6; ++i)
    if (ptrs[i]) PSA_TRY(check_aligned(fn, names[i], ptrs[i]));
  const int64_t eb = elt_bytes(dtype);
  const int64_t nq = static_cast<int64_t>(BH) * n_q * head_dim;
  const int64_t nk = static_cast<int64_t>(BH) * n_k * head_dim;
  const Range outs[3] = {range("o", o, nq, eb), range("lse", lse, static_cast<int64_t>(BH) * n_q, 4),
                         range("workspace", workspace, workspace ? static_cast<int64_t>(workspace_bytes) : 0, 1)};
  const Range ins[3] = {range("q", q, nq, eb), range("k", k, nk, eb), range("v", v, nk, eb)};
  for (const Range& a : outs)
    for (const Range& b : ins) {
      const Range pair[2] = {a, b};
      PSA_TRY(check_disjoint(fn, pair, 2));
    }
  PSA_TRY(check_disjoint(fn, outs, 3));
  return launched(fn, [&] {
    return psa::launch_fa2_fwd(q, k, v, o, lse, BH, n_q, n_k, head_dim, scale, dtype == PSA_BF16,
                               workspace, workspace ? workspace_bytes : 0, as_stream(stream));
  });
}

size_t fa2_bwd_workspace_bytes(int BH, int n_q) {
  if (BH <= 0 || n_q <= 0) return 0;
  return 2 * static_cast<size_t>(BH) * static_cast<size_t>(n_q) * sizeof(float);
}

psa_status fa2_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv, float* workspace, int BH,
                   int n_q, int n_k, int head_dim, float scale, psa_dtype dtype, void* stream) {
  const char* fn = "fa2_bwd";
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !workspace)
    return fail(PSA_ERR_NULL, fn, "every pointer argument is required");
  PSA_TRY(check_attn(fn, BH, n_q, n_k, head_dim, scale, dtype));
  const char* names[10] = {"q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv", "workspace"};
  const void* ptrs[10] = {q, k, v, o, dout, lse, dq, dk, dv, workspace};
  for (int i = 0; i < 10; ++i) PSA_TRY(check_aligned(fn, names[i], ptrs[i]));
  const int64_t eb = elt_bytes(dtype);
  const int64_t nq = static_cast<int64_t>(BH) * n_q * head_dim;
  const int64_t nk = static_cast<int64_t>(BH) * n_k * head_dim;
  const int64_t rows = static_cast<int64_t>(BH) * n_q;
  const Range outs[4] = {range("dq", dq, nq, eb), range("dk", dk, nk, eb), range("dv", dv, nk, eb),
                         range("workspace", workspace, 2 * rows, 4)};
  const Range ins[6] = {range("q", q, nq, eb),  range("k", k, nk, eb),
                        range("v", v, nk, eb),  range("o", o, nq, eb),
                        range("dout", dout, nq, eb), range("lse", lse, rows, 4)};
  PSA_TRY(check_disjoint(fn, outs, 4));
  for (const Range& a : outs)
    for (const Range& b : ins) {
      const Range pair[2] = {a, b};
      PSA_TRY(check_disjoint(fn, pair, 2));
    }
  return launched(fn, [&] {
    return psa::launch_fa2_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace, BH, n_q, n_k, head_dim,
                               scale, dtype == PSA_BF16, as_stream(stream));
  });
}

psa_status fa2_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* lse, void* dq, void* dk, void* dv,
                           int BH, int n_q, int n_k, int head_dim, float scale, psa_dtype dtype,
                           void* stream) {
  const char* fn = "fa2_bwd_noalloc";
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv)
    return fail(PSA_ERR_NULL, fn, "every pointer argument is required");
  PSA_TRY(check_attn(fn, BH, n_q, n_k, head_dim, scale, dtype));
  const int64_t rows = static_cast<int64_t>(BH) * n_q;
  if (rows > static_cast<int64_t>(PSA_NOALLOC_SCRATCH_BYTES / (2 * sizeof(float))))
    return fail(PSA_ERR_SHAPE, fn,
                "BH*n_q=%lld rows need %lld bytes of scratch; the limit is %lld bytes "
                "(BH*n_q <= %lld): call fa2_bwd with a workspace instead",
                static_cast<long long>(rows), static_cast<long long>(rows * 8),
                static_cast<long long>(PSA_NOALLOC_SCRATCH_BYTES),
                static_cast<long long>(PSA_NOALLOC_SCRATCH_BYTES / (2 * sizeof(float))));
  const char* names[9] = {"q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv"};
  const void* ptrs[9] = {q, k, v, o, dout, lse, dq, dk, dv};
  for (int i = 0; i < 9; ++i) PSA_TRY(check_aligned(fn, names[i], ptrs[i]));
  const int64_t eb = elt_bytes(dtype);
  const int64_t nq = static_cast<int64_t>(BH) * n_q * head_dim;
  const int64_t nk = static_cast<int64_t>(BH) * n_k * head_dim;
  const Range outs[3] = {range("dq", dq, nq, eb), range("dk", dk, nk, eb), range("dv", dv, nk, eb)};
  const Range ins[6] = {range("q", q, nq, eb),  range("k", k, nk, eb),
                        range("v", v, nk, eb),  range("o", o, nq, eb),
                        range("dout", dout, nq, eb), range("lse", lse, rows, 4)};
  PSA_TRY(check_disjoint(fn, outs, 3));
  for (const Range& a : outs)
    for (const Range& b : ins) {
      const Range pair[2] = {a, b};
      PSA_TRY(check_disjoint(fn, pair, 2));
    }
  return launched(fn, [&] {
    return psa::launch_fa2_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, BH, n_q, n_k, head_dim,
                                       scale, dtype == PSA_BF16, as_stream(stream));
  });
}

size_t psa_attention_fwd_workspace_bytes(int B, int heads, int key_dim, int H, int W,
                                         psa_dtype dtype) {
  if (B <= 0 || heads <= 0 || H <= 0 || W <= 0 || !supported_dim(key_dim) ||
      (dtype != PSA_F32 && dtype != PSA_BF16))
    return 0;
  const int64_t N = static_cast<int64_t>(H) * W;
  const int64_t BH = static_cast<int64_t>(B) * heads;
  if (N > (1 << 28) || BH > (1 << 24)) return 0;
  return psa::psa_fused_split_bytes(static_cast<int>(BH), key_dim, static_cast<int>(N),
                                    dtype == PSA_BF16);
}

psa_status psa_attention_fwd(const void* qkv_nchw, void* out_nchw, void* v_nchw, float* lse, int B,
                             int heads, int key_dim, int H, int W, float scale, psa_dtype dtype,
                             void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "psa_attention_fwd";
  if (!qkv_nchw) return fail(PSA_ERR_NULL, fn, "qkv_nchw is NULL");
  if (!out_nchw) return fail(PSA_ERR_NULL, fn, "out_nchw is NULL");
  PSA_TRY(check_map(fn, B, heads, key_dim, H, W, dtype));
  PSA_TRY(check_launch_rows(fn, static_cast<int64_t>(B) * heads, static_cast<int64_t>(H) * W));
  if (!std::isfinite(scale) || !(scale > 0.0f))
    return fail(PSA_ERR_UNSUPPORTED, fn, "scale=%g must be finite and > 0", static_cast<double>(scale));
  PSA_TRY(check_aligned(fn, "qkv_nchw", qkv_nchw));
  PSA_TRY(check_aligned(fn, "out_nchw", out_nchw));
  if (v_nchw) PSA_TRY(check_aligned(fn, "v_nchw", v_nchw));
  if (lse) PSA_TRY(check_aligned(fn, "lse", lse));
  if (workspace) PSA_TRY(check_aligned(fn, "workspace", workspace));
  const int64_t eb = elt_bytes(dtype);
  const int64_t half = static_cast<int64_t>(B) * heads * key_dim * H * W;  // elements per [., KD] set
  const Range r[5] = {range("qkv_nchw", qkv_nchw, 4 * half, eb),
                      range("out_nchw", out_nchw, 2 * half, eb),
                      range("v_nchw", v_nchw, v_nchw ? 2 * half : 0, eb),
                      range("lse", lse, lse ? static_cast<int64_t>(B) * heads * H * W : 0, 4),
                      range("workspace", workspace, workspace ? static_cast<int64_t>(workspace_bytes) : 0, 1)};
  PSA_TRY(check_disjoint(fn, r, 5));
  return launched(fn, [&] {
    return psa::launch_psa_fused_fwd(qkv_nchw, out_nchw, v_nchw, lse, B * heads, key_dim, H * W,
                                     scale, dtype == PSA_BF16, workspace, workspace ?
                                     workspace_bytes : 0, as_stream(stream));
  });
}

size_t psa_attention_bwd_workspace_bytes(int B, int heads, int H, int W) {
  if (B <= 0 || heads <= 0 || H <= 0 || W <= 0) return 0;
  return 2 * static_cast<size_t>(B) * heads * H * W * sizeof(float);
}

psa_status psa_attention_bwd(const void* qkv_nchw, const void* out_nchw, const float* lse,
                             const void* dout_nchw, const void* dv_nchw, void* dqkv_nchw,
                             float* workspace, int B, int heads, int key_dim, int H, int W,
                             float scale, psa_dtype dtype, void* stream) {
  const char* fn = "psa_attention_bwd";
  if (!qkv_nchw || !out_nchw || !lse || !dout_nchw || !dqkv_nchw || !workspace)
    return fail(PSA_ERR_NULL, fn, "qkv_nchw, out_nchw, lse, dout_nchw, dqkv_nchw and workspace "
                                  "must not be NULL (dv_nchw may be)");
  PSA_TRY(check_map(fn, B, heads, key_dim, H, W, dtype));
  PSA_TRY(check_launch_rows(fn, static_cast<int64_t>(B) * heads, static_cast<int64_t>(H) * W));
  if (!std::isfinite(scale) || !(scale > 0.0f))
    return fail(PSA_ERR_UNSUPPORTED, fn, "scale=%g must be finite and > 0", static_cast<double>(scale));
  const char* names[7] = {"qkv_nchw", "out_nchw", "lse", "dout_nchw", "dv_nchw", "dqkv_nchw", "workspace"};
  const void* ptrs[7] = {qkv_nchw, out_nchw, lse, dout_nchw, dv_nchw, dqkv_nchw, workspace};
  for (int i = 0; i < 7; ++i)
    if (ptrs[i]) PSA_TRY(check_aligned(fn, names[i], ptrs[i]));
  const int64_t eb = elt_bytes(dtype);
  const int64_t half = static_cast<int64_t>(B) * heads * key_dim * H * W;
  const int64_t rows = static_cast<int64_t>(B) * heads * H * W;
  const Range outs[2] = {range("dqkv_nchw", dqkv_nchw, 4 * half, eb),
                         range("workspace", workspace, 2 * rows, 4)};
  const Range ins[5] = {range("qkv_nchw", qkv_nchw, 4 * half, eb), range("out_nchw", out_nchw, 2 * half, eb),
                        range("lse", lse, rows, 4), range("dout_nchw", dout_nchw, 2 * half, eb),
                        range("dv_nchw", dv_nchw, dv_nchw ? 2 * half : 0, eb)};
  PSA_TRY(check_disjoint(fn, outs, 2));
  for (const Range& a : outs)
    for (const Range& b : ins) {
      const Range pair[2] = {a, b};
      PSA_TRY(check_disjoint(fn, pair, 2));
    }
  return launched(fn, [&] {
    return psa::launch_psa_fused_bwd(qkv_nchw, out_nchw, lse, dout_nchw, dv_nchw, dqkv_nchw,
                                     workspace, B * heads, key_dim, H * W, scale, dtype == PSA_BF16,
                                     as_stream(stream));
  });
}

psa_status detect_decode(const void* boxes, const float* anchor_x, const float* anchor_y,
                         const float* strides, void* out, int B, long long A, psa_dtype dtype,
                         void* stream) {
  const char* fn = "detect_decode";
  if (!boxes) return fail(PSA_ERR_NULL, fn, "boxes is NULL");
  if (!anchor_x) return fail(PSA_ERR_NULL, fn, "anchor_x is NULL");
  if (!anchor_y) return fail(PSA_ERR_NULL, fn, "anchor_y is NULL");
  if (!strides) return fail(PSA_ERR_NULL, fn, "strides is NULL");
  if (!out) return fail(PSA_ERR_NULL, fn, "out is NULL");
  if (B <= 0 || A <= 0)
    return fail(PSA_ERR_SHAPE, fn, "dims must be > 0 (B=%d A=%lld)", B, A);
  // The batch item is the grid's y index; anchor tiles are the x index.
  // A grid dimension holds fewer than 2^32 work-items, so the anchor count stays below 2^31.
  if (B > 65535 || A > kMaxLanes || static_cast<int64_t>(B) * 4 * A > (int64_t(1) << 40))
    return fail(PSA_ERR_SHAPE, fn, "sizes too large (B=%d A=%lld)", B, A);
  PSA_TRY(check_dtype(fn, dtype));
  const void* ptrs[5] = {boxes, anchor_x, anchor_y, strides, out};
  const char* names[5] = {"boxes", "anchor_x", "anchor_y", "strides", "out"};
  for (int i = 0; i < 5; ++i) PSA_TRY(check_aligned(fn, names[i], ptrs[i]));
  const int64_t n = static_cast<int64_t>(B) * 4 * A;
  const Range r[5] = {range("boxes", boxes, n, elt_bytes(dtype)), range("anchor_x", anchor_x, A, 4),
                      range("anchor_y", anchor_y, A, 4), range("strides", strides, A, 4),
                      range("out", out, n, elt_bytes(dtype))};
  PSA_TRY(check_outputs_disjoint(fn, r, 5, 4));
  return launched(fn, [&] {
    return psa::launch_detect_decode(boxes, anchor_x, anchor_y, strides, out, B, A, dtype ==
                                     PSA_BF16, as_stream(stream));
  });
}

psa_status ciou_loss_fwd(const float* pred, const float* target, float* loss, float* iou,
                         float* v, float* alpha, long long N, void* stream) {
  const char* fn = "ciou_loss_fwd";
  const void* ptrs[6] = {pred, target, loss, iou, v, alpha};
  const char* names[6] = {"pred", "target", "loss", "iou", "v", "alpha"};
  for (int i = 0; i < 6; ++i)
    if (!ptrs[i]) return fail(PSA_ERR_NULL, fn, "%s is NULL", names[i]);
  if (N <= 0) return fail(PSA_ERR_SHAPE, fn, "N=%lld must be > 0", N);
  if (N > kMaxLanes) return fail(PSA_ERR_SHAPE, fn, "N=%lld too large", N);
  for (int i = 0; i < 6; ++i) PSA_TRY(check_aligned(fn, names[i], ptrs[i]));
  const Range r[6] = {range("pred", pred, 4 * N, 4), range("target", target, 4 * N, 4),
                      range("loss", loss, N, 4),     range("iou", iou, N, 4),
                      range("v", v, N, 4),           range("alpha", alpha, N, 4)};
  PSA_TRY(check_outputs_disjoint(fn, r, 6, 2));
  return launched(fn, [&] {
    return psa::launch_ciou_fwd(pred, target, loss, iou, v, alpha, N, as_stream(stream));
  });
}

psa_status ciou_loss_bwd(const float* pred, const float* target, const float* iou,
                         const float* v, const float* alpha, const float* dloss, float* dpred,
                         long long N, void* stream) {
  const char* fn = "ciou_loss_bwd";
  const void* ptrs[7] = {pred, target, iou, v, alpha, dloss, dpred};
  const char* names[7] = {"pred", "target", "iou", "v", "alpha", "dloss", "dpred"};
  for (int i = 0; i < 7; ++i)
    if (!ptrs[i]) return fail(PSA_ERR_NULL, fn, "%s is NULL", names[i]);
  if (N <= 0) return fail(PSA_ERR_SHAPE, fn, "N=%lld must be > 0", N);
  if (N > kMaxLanes) return fail(PSA_ERR_SHAPE, fn, "N=%lld too large", N);
  for (int i = 0; i < 7; ++i) PSA_TRY(check_aligned(fn, names[i], ptrs[i]));
  const Range r[7] = {range("pred", pred, 4 * N, 4), range("target", target, 4 * N, 4),
                      range("iou", iou, N, 4),         range("v", v, N, 4),
                      range("alpha", alpha, N, 4),     range("dloss", dloss, N, 4),
                      range("dpred", dpred, 4 * N, 4)};
  PSA_TRY(check_outputs_disjoint(fn, r, 7, 6));
  return launched(fn, [&] {
    return psa::launch_ciou_bwd(pred, target, iou, v, alpha, dloss, dpred, N, as_stream(stream));
  });
}

const char* psa_last_error(void) { return g_last_error.c_str(); }

int psa_abi_version(void) { return PSA_ABI_VERSION; }

}  // extern "C"
