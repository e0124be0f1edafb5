// C ABI of libmoe.so: argument checks on the host, then kernel launches on the
// caller's stream.  Nothing here allocates device memory or synchronises.
#include <stdarg.h>
#include <stdio.h>

#include <cmath>

#include "moe_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = '\0';
  return MOE_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define NEED_PTR(p)                                                                 \
  do {                                                                              \
    if ((p) == nullptr) return fail(MOE_ERR_INVALID_ARG, "%s is NULL", #p);         \
    if (!aligned16(p)) return fail(MOE_ERR_INVALID_ARG, "%s is not 16-byte aligned", #p); \
  } while (0)

#define OPT_PTR(p)                                                                  \
  do {                                                                              \
    if ((p) != nullptr && !aligned16(p))                                            \
      return fail(MOE_ERR_INVALID_ARG, "%s is not 16-byte aligned", #p);            \
  } while (0)

// Shape checks common to every entry point.
int check_shape(const moe_shape* s) {
  if (s == nullptr) return fail(MOE_ERR_INVALID_ARG, "shape is NULL");
  if (s->dtype != MOE_F32 && s->dtype != MOE_BF16)
    return fail(MOE_ERR_INVALID_ARG, "dtype %d is neither MOE_F32 nor MOE_BF16", s->dtype);
  if (s->T < 0) return fail(MOE_ERR_INVALID_ARG, "T = %d < 0", s->T);
  if (s->E < 1) return fail(MOE_ERR_INVALID_ARG, "E = %d < 1", s->E);
  if (s->k < 1 || s->k > s->E) return fail(MOE_ERR_INVALID_ARG, "k = %d outside 1..E (E = %d)", s->k, s->E);
  if (s->D < 1 || s->F < 1 || s->Fs < 0)
    return fail(MOE_ERR_INVALID_ARG, "D = %d, F = %d, Fs = %d: widths must be positive (Fs >= 0)", s->D, s->F, s->Fs);
  if (!std::isfinite(s->alpha)) return fail(MOE_ERR_INVALID_ARG, "alpha is not finite");
  if (s->E > 256) return fail(MOE_ERR_UNSUPPORTED, "E = %d > 256", s->E);
  if (s->k > 16) return fail(MOE_ERR_UNSUPPORTED, "k = %d > 16", s->k);
  if (static_cast<int64_t>(s->T) * s->k >= (int64_t{1} << 31))
    return fail(MOE_ERR_UNSUPPORTED, "k*T = %lld does not fit int32", static_cast<long long>(s->T) * s->k);
  if (s->dtype == MOE_BF16) {
    if (s->D % 256 != 0) return fail(MOE_ERR_UNSUPPORTED, "bf16: D = %d is not a multiple of 256", s->D);
    // every GEMM reduction (D, F, Fs) is a whole number of 256-wide weight
    // prefetch rounds; output tiles are 128 (gate/up) and 256 (down) wide
    if (s->F % 256 != 0) return fail(MOE_ERR_UNSUPPORTED, "bf16: F = %d is not a multiple of 256", s->F);
    if (s->Fs % 256 != 0) return fail(MOE_ERR_UNSUPPORTED, "bf16: Fs = %d is not a multiple of 256", s->Fs);
    // token rows are addressed by 32-bit byte offsets
    if (static_cast<int64_t>(s->T) * s->D * 2 >= (int64_t{1} << 32) ||
        static_cast<int64_t>(s->T) * s->Fs * 2 >= (int64_t{1} << 32))
      return fail(MOE_ERR_UNSUPPORTED, "bf16: T * D and T * Fs must stay below 2^31");
  } else {
    if (s->D % 32 != 0 || s->F % 16 != 0 || s->Fs % 16 != 0)
      return fail(MOE_ERR_UNSUPPORTED, "fp32: D must be a multiple of 32, F and Fs of 16");
    if (s->D > 8192 || s->F > 8192 || s->Fs > 8192)
      return fail(MOE_ERR_UNSUPPORTED, "fp32: D, F and Fs are limited to 8192");
  }
  return MOE_OK;
}

int launched(hipError_t e) {
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

int moe_version(void) { return 1; }

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

const char* moe_last_error(void) { return g_err; }

size_t moe_workspace_bytes(const moe_shape* shape) {
  if (check_shape(shape) != MOE_OK) return 0;
  return moe::permute_workspace_bytes(*shape);
}

int moe_route_masked(const moe_shape* shape, const void* x, const void* w_router, const float* bias,
                     const uint8_t* mask, float* logits, int32_t* topk_idx, float* topk_w,
                     void* stream) {
  if (int r = check_shape(shape)) return r;
  if (shape->T == 0) return ok();
  NEED_PTR(x);
  NEED_PTR(w_router);
  OPT_PTR(bias);
  NEED_PTR(logits);
  NEED_PTR(topk_idx);
  NEED_PTR(topk_w);
  const moe_shape& s = *shape;
  if (s.dtype == MOE_BF16)
    return launched(moe::launch_route_bf16(s, static_cast<const moe::bf16_t*>(x),
                                           static_cast<const moe::bf16_t*>(w_router), bias, mask,
                                           logits, topk_idx, topk_w, as_stream(stream)));
  return launched(moe::launch_route_f32(s, static_cast<const float*>(x),
                                        static_cast<const float*>(w_router), bias, mask, logits,
                                        topk_idx, topk_w, as_stream(stream)));
}

int moe_route(const moe_shape* shape, const void* x, const void* w_router, const float* bias,
              float* logits, int32_t* topk_idx, float* topk_w, void* stream) {
  return moe_route_masked(shape, x, w_router, bias, nullptr, logits, topk_idx, topk_w, stream);
}

int moe_permute(const moe_shape* shape, const int32_t* topk_idx, const void* x, int32_t* counts,
                int32_t* offsets, int32_t* sorted_token, int32_t* slot_of, void* x_perm,
                void* workspace, size_t workspace_bytes, void* stream) {
  if (int r = check_shape(shape)) return r;
  if (shape->T == 0) return ok();
  NEED_PTR(topk_idx);
  NEED_PTR(counts);
  NEED_PTR(offsets);
  NEED_PTR(sorted_token);
  NEED_PTR(slot_of);
  OPT_PTR(x_perm);
  if (x_perm) NEED_PTR(x);
  if (workspace == nullptr || !aligned16(workspace))
    return fail(MOE_ERR_WORKSPACE, "workspace is NULL or not 16-byte aligned");
  const size_t need = moe::permute_workspace_bytes(*shape);
  if (workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", workspace_bytes, need);
  return launched(moe::launch_permute(*shape, topk_idx, x, counts, offsets, sorted_token, slot_of,
                                      x_perm, workspace, as_stream(stream)));
}

int moe_permute_static(const moe_shape* shape, const int32_t* topk_idx, const void* x, int32_t* counts,
                       int32_t* offsets, int32_t* sorted_token, int32_t* slot_of, void* x_perm,
                       void* stream) {
  if (int r = check_shape(shape)) return r;
  if (shape->T == 0) return ok();
  NEED_PTR(topk_idx);
  NEED_PTR(counts);
  NEED_PTR(offsets);
  NEED_PTR(sorted_token);
  NEED_PTR(slot_of);
  OPT_PTR(x_perm);
  if (x_perm) NEED_PTR(x);
  const size_t need = moe::permute_workspace_bytes(*shape);
  if (need > moe::static_scratch_bytes())
    return fail(MOE_ERR_UNSUPPORTED, "moe_permute_static: %zu bytes of scratch needed, %zu available "
                "(T = %d, E = %d); use moe_permute with a workspace", need, moe::static_scratch_bytes(),
                shape->T, shape->E);
  void* scratch = nullptr;
  if (hipError_t e = moe::static_scratch(&scratch))
    return fail(MOE_ERR_HIP, "moe_permute_static: scratch address lookup failed: %s", hipGetErrorString(e));
  return launched(moe::launch_permute(*shape, topk_idx, x, counts, offsets, sorted_token, slot_of,
                                      x_perm, scratch, as_stream(stream)));
}

int moe_grouped_gate_up(const moe_shape* shape, const void* x_perm, const int32_t* sorted_token,
                        const void* x, const int32_t* offsets, const void* w_gate_up,
                        const void* ws_gate_up, void* h, void* stream) {
  if (int r = check_shape(shape)) return r;
  if (shape->T == 0) return ok();
  OPT_PTR(x_perm);
  if (x_perm == nullptr) NEED_PTR(sorted_token);
  NEED_PTR(x);
  NEED_PTR(offsets);
  NEED_PTR(w_gate_up);
  if (shape->Fs > 0 && shape->dtype != MOE_BF16) NEED_PTR(ws_gate_up);
  NEED_PTR(h);
  const moe_shape& s = *shape;
  if (s.dtype == MOE_BF16)
    return launched(moe::launch_gate_up_bf16(
        s, static_cast<const moe::bf16_t*>(x_perm), sorted_token, static_cast<const moe::bf16_t*>(x),
        offsets, static_cast<const moe::bf16_t*>(w_gate_up),
        static_cast<const moe::bf16_t*>(ws_gate_up), static_cast<moe::bf16_t*>(h), as_stream(stream)));
  return launched(moe::launch_gate_up_f32(s, static_cast<const float*>(x_perm), sorted_token,
                                          static_cast<const float*>(x), offsets,
                                          static_cast<const float*>(w_gate_up),
                                          static_cast<const float*>(ws_gate_up),
                                          static_cast<float*>(h), as_stream(stream)));
}

int moe_grouped_down(const moe_shape* shape, const void* h, const int32_t* offsets,
                     const void* w_down, const void* ws_down, void* y_perm, void* y_shared,
                     void* stream) {
  if (int r = check_shape(shape)) return r;
  if (shape->T == 0) return ok();
  NEED_PTR(h);
  NEED_PTR(offsets);
  NEED_PTR(w_down);
  NEED_PTR(y_perm);
  if (shape->Fs > 0 && (shape->dtype != MOE_BF16 || ws_down != nullptr)) {
    NEED_PTR(ws_down);
    NEED_PTR(y_shared);
  }
  const moe_shape& s = *shape;
  if (s.dtype == MOE_BF16)
    return launched(moe::launch_down_bf16(
        s, static_cast<const moe::bf16_t*>(h), offsets, static_cast<const moe::bf16_t*>(w_down),
        static_cast<const moe::bf16_t*>(ws_down), static_cast<moe::bf16_t*>(y_perm),
        static_cast<moe::bf16_t*>(y_shared), as_stream(stream)));
  return launched(moe::launch_down_f32(s, static_cast<const float*>(h), offsets,
                                       static_cast<const float*>(w_down),
                                       static_cast<const float*>(ws_down),
                                       static_cast<float*>(y_perm), static_cast<float*>(y_shared),
                                       as_stream(stream)));
}

int moe_shared_ffn(const moe_shape* shape, const void* x, const void* ws_gate_up,
                   const void* ws_down, void* h_shared, void* y_shared, void* stream) {
  if (int r = check_shape(shape)) return r;
  if (shape->dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "moe_shared_ffn: bf16 only");
  if (shape->Fs == 0) return fail(MOE_ERR_INVALID_ARG, "moe_shared_ffn: no shared expert (Fs = 0)");
  if (shape->T == 0) return ok();
  NEED_PTR(x);
  NEED_PTR(ws_gate_up);
  NEED_PTR(ws_down);
  NEED_PTR(h_shared);
  NEED_PTR(y_shared);
  return launched(moe::launch_shared_ffn_bf16(
      *shape, static_cast<const moe::bf16_t*>(x), static_cast<const moe::bf16_t*>(ws_gate_up),
      static_cast<const moe::bf16_t*>(ws_down), static_cast<moe::bf16_t*>(h_shared),
      static_cast<moe::bf16_t*>(y_shared), as_stream(stream)));
}

int moe_grouped_ffn(const moe_shape* shape, const void* x_perm, const int32_t* sorted_token,
                    const void* x, const int32_t* offsets, const void* w_gate_up,
                    const void* w_down, const void* ws_gate_up, const void* ws_down, void* h,
                    void* y_perm, void* y_shared, void* stream) {
  if (int r = check_shape(shape)) return r;
  if (shape->T == 0) return ok();
  // check both halves before launching either
  OPT_PTR(x_perm);
  if (x_perm == nullptr) NEED_PTR(sorted_token);
  NEED_PTR(x);
  NEED_PTR(offsets);
  NEED_PTR(w_gate_up);
  NEED_PTR(w_down);
  NEED_PTR(h);
  NEED_PTR(y_perm);
  if (shape->Fs > 0) {
    NEED_PTR(ws_gate_up);
    NEED_PTR(ws_down);
    NEED_PTR(y_shared);
  }
  if (int r = moe_grouped_gate_up(shape, x_perm, sorted_token, x, offsets, w_gate_up, ws_gate_up,
                                  h, stream))
    return r;
  return moe_grouped_down(shape, h, offsets, w_down, ws_down, y_perm, y_shared, stream);
}

size_t moe_packed_bytes(int64_t count, int32_t rows, int32_t cols, int32_t dtype) {
  if ((dtype != MOE_F32 && dtype != MOE_BF16) || count < 0 || rows < 0 || cols < 0 || rows % 32 != 0 ||
      cols % 16 != 0)
    return 0;
  return static_cast<size_t>(count) * moe::packed_matrix_elems(rows, cols) * (dtype == MOE_BF16 ? 2 : 4);
}

int moe_pack_weights(const void* w, void* w_packed, int64_t count, int32_t rows, int32_t cols,
                     int32_t dtype, void* stream) {
  if (dtype != MOE_F32 && dtype != MOE_BF16)
    return fail(MOE_ERR_INVALID_ARG, "dtype %d is neither MOE_F32 nor MOE_BF16", dtype);
  if (count < 0 || rows < 0 || cols < 0)
    return fail(MOE_ERR_INVALID_ARG, "negative count or size");
  if (rows % 32 != 0 || cols % 16 != 0)
    return fail(MOE_ERR_INVALID_ARG, "rows = %d must be a multiple of 32 and cols = %d of 16", rows, cols);
  if (count == 0 || rows == 0 || cols == 0) return ok();
  NEED_PTR(w);
  NEED_PTR(w_packed);
  const int elem = dtype == MOE_BF16 ? 2 : 4;
  const uintptr_t a = reinterpret_cast<uintptr_t>(w), b = reinterpret_cast<uintptr_t>(w_packed);
  const uintptr_t in_bytes = static_cast<uintptr_t>(count) * rows * cols * elem;
  const uintptr_t out_bytes = moe_packed_bytes(count, rows, cols, dtype);
  if (a < b + out_bytes && b < a + in_bytes) return fail(MOE_ERR_INVALID_ARG, "w and w_packed overlap");
  return launched(moe::launch_pack(w, w_packed, count, rows, cols, elem, as_stream(stream)));
}

size_t moe_fp8_packed_bytes(int64_t count, int32_t rows, int32_t cols) {
  if (count < 0 || rows < 0 || cols < 0 || rows % 32 != 0 || cols % 32 != 0) return 0;
  return static_cast<size_t>(count) * rows * cols;
}

int moe_quantize_weights_fp8(const void* w, void* w_fp8, float* scales, int64_t count, int32_t rows,
                             int32_t cols, void* stream) {
  if (count < 0 || rows < 0 || cols < 0) return fail(MOE_ERR_INVALID_ARG, "negative count or size");
  if (rows % 32 != 0 || cols % 32 != 0)
    return fail(MOE_ERR_INVALID_ARG, "rows = %d and cols = %d must be multiples of 32", rows, cols);
  if (count == 0 || rows == 0 || cols == 0) return ok();
  NEED_PTR(w);
  NEED_PTR(w_fp8);
  NEED_PTR(scales);
  const uintptr_t a = reinterpret_cast<uintptr_t>(w), b = reinterpret_cast<uintptr_t>(w_fp8),
                  c = reinterpret_cast<uintptr_t>(scales);
  const uintptr_t na = static_cast<uintptr_t>(count) * rows * cols * 2;
  const uintptr_t nb = moe_fp8_packed_bytes(count, rows, cols);
  const uintptr_t nc = static_cast<uintptr_t>(count) * rows * 4;
  if ((a < b + nb && b < a + na) || (a < c + nc && c < a + na) || (b < c + nc && c < b + nb))
    return fail(MOE_ERR_INVALID_ARG, "w, w_fp8 and scales overlap");
  return launched(moe::launch_quantize_fp8(w, w_fp8, scales, count, rows, cols, as_stream(stream)));
}

int moe_grouped_gate_up_fp8(const moe_shape* shape, const void* x_perm, const int32_t* sorted_token,
                            const void* x, const int32_t* offsets, const void* w_gate_up,
                            const float* w_gate_up_scale, const void* ws_gate_up,
                            const float* ws_gate_up_scale, void* h, void* stream) {
  if (int r = check_shape(shape)) return r;
  if (shape->dtype != MOE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "FP8 weights need bf16 activations (dtype MOE_BF16)");
  if (shape->T == 0) return ok();
  OPT_PTR(x_perm);
  if (x_perm == nullptr) NEED_PTR(sorted_token);
  NEED_PTR(x);
  NEED_PTR(offsets);
  NEED_PTR(w_gate_up);
  NEED_PTR(w_gate_up_scale);
  if (shape->Fs > 0) {
    NEED_PTR(ws_gate_up);
    NEED_PTR(ws_gate_up_scale);
  }
  NEED_PTR(h);
  const moe_shape& s = *shape;
  return launched(moe::launch_gate_up_fp8(
      s, static_cast<const moe::bf16_t*>(x_perm), sorted_token, static_cast<const moe::bf16_t*>(x),
      offsets, static_cast<const uint8_t*>(w_gate_up), w_gate_up_scale,
      static_cast<const uint8_t*>(ws_gate_up), ws_gate_up_scale, static_cast<moe::bf16_t*>(h),
      as_stream(stream)));
}

int moe_grouped_down_fp8(const moe_shape* shape, const void* h, const int32_t* offsets,
                         const void* w_down, const float* w_down_scale, const void* ws_down,
                         const float* ws_down_scale, void* y_perm, void* y_shared, void* stream) {
  if (int r = check_shape(shape)) return r;
  if (shape->dtype != MOE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "FP8 weights need bf16 activations (dtype MOE_BF16)");
  if (shape->T == 0) return ok();
  NEED_PTR(h);
  NEED_PTR(offsets);
  NEED_PTR(w_down);
  NEED_PTR(w_down_scale);
  NEED_PTR(y_perm);
  if (shape->Fs > 0) {
    NEED_PTR(ws_down);
    NEED_PTR(ws_down_scale);
    NEED_PTR(y_shared);
  }
  const moe_shape& s = *shape;
  return launched(moe::launch_down_fp8(
      s, static_cast<const moe::bf16_t*>(h), offsets, static_cast<const uint8_t*>(w_down),
      w_down_scale, static_cast<const uint8_t*>(ws_down), ws_down_scale,
      static_cast<moe::bf16_t*>(y_perm), static_cast<moe::bf16_t*>(y_shared), as_stream(stream)));
}

int moe_combine(const moe_shape* shape, const void* y_perm, const void* y_shared,
                const int32_t* slot_of, const float* topk_w, void* out, void* stream) {
  if (int r = check_shape(shape)) return r;
  if (shape->T == 0) return ok();
  NEED_PTR(y_perm);
  OPT_PTR(y_shared);
  NEED_PTR(slot_of);
  NEED_PTR(topk_w);
  NEED_PTR(out);
  return launched(moe::launch_combine(*shape, y_perm, y_shared, slot_of, topk_w, out,
                                      as_stream(stream)));
}

// ------------------------------------------------------------ training pass

size_t moe_train_workspace_bytes(const moe_shape* shape) {
  if (check_shape(shape) != MOE_OK) return 0;
  return moe::train_workspace_bytes(*shape);
}

size_t moe_packed_transposed_bytes(int64_t count, int32_t rows, int32_t cols, int32_t k_padded) {
  if (count < 0 || rows < 0 || cols < 0 || cols % 32 != 0 || k_padded % 16 != 0 || k_padded < rows)
    return 0;
  return static_cast<size_t>(count) * cols * k_padded * 2;
}

int moe_pack_weights_transposed(const void* w, void* w_packed, int64_t count, int32_t rows, int32_t cols,
                                int32_t k_padded, void* stream) {
  if (count < 0 || rows < 0 || cols < 0) return fail(MOE_ERR_INVALID_ARG, "negative count or size");
  if (cols % 32 != 0 || k_padded % 16 != 0 || k_padded < rows)
    return fail(MOE_ERR_INVALID_ARG,
                "cols = %d must be a multiple of 32, k_padded = %d a multiple of 16 and >= rows = %d", cols,
                k_padded, rows);
  if (count == 0 || cols == 0 || k_padded == 0) return ok();
  NEED_PTR(w_packed);
  if (rows > 0) NEED_PTR(w);
  const uintptr_t a = reinterpret_cast<uintptr_t>(w), b = reinterpret_cast<uintptr_t>(w_packed);
  const uintptr_t in_bytes = static_cast<uintptr_t>(count) * rows * cols * 2;
  const uintptr_t out_bytes = moe_packed_transposed_bytes(count, rows, cols, k_padded);
  if (rows > 0 && a < b + out_bytes && b < a + in_bytes)
    return fail(MOE_ERR_INVALID_ARG, "w and w_packed overlap");
  return launched(moe::launch_pack_transposed(w, w_packed, count, rows, cols, k_padded, as_stream(stream)));
}

namespace {
int check_train_shape(const moe_shape* shape) {
  if (int r = check_shape(shape)) return r;
  if (shape->dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "the training pass is bf16 only");
  // the shared expert's [dg | du] rows (2 Fs wide) are addressed by 32-bit byte offsets
  if (static_cast<int64_t>(shape->T) * 2 * shape->Fs * 2 >= (int64_t{1} << 32))
    return fail(MOE_ERR_UNSUPPORTED, "training: T * 2 Fs must stay below 2^31");
  return MOE_OK;
}

int check_workspace(void* ws, size_t ws_bytes, size_t need) {
  if (ws == nullptr || !aligned16(ws)) return fail(MOE_ERR_WORKSPACE, "workspace is NULL or not 16-byte aligned");
  if (ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", ws_bytes, need);
  return MOE_OK;
}
}  // namespace

int moe_load_stats(const moe_shape* shape, const float* logits, const int32_t* topk_idx,
                   const int32_t* counts, const int32_t* counts_global, float beta, float* f, float* p,
                   float* aux_loss, float* aux_coef, void* workspace, size_t workspace_bytes,
                   void* stream) {
  if (int r = check_shape(shape)) return r;
  if (!std::isfinite(beta)) return fail(MOE_ERR_INVALID_ARG, "beta is not finite");
  NEED_PTR(counts);
  OPT_PTR(counts_global);
  NEED_PTR(f);
  NEED_PTR(p);
  NEED_PTR(aux_loss);
  NEED_PTR(aux_coef);
  if (shape->T > 0) {
    NEED_PTR(logits);
    NEED_PTR(topk_idx);
  }
  if (int r = check_workspace(workspace, workspace_bytes, moe::train_workspace_bytes(*shape))) return r;
  return launched(moe::launch_load_stats(*shape, logits, topk_idx, counts, counts_global, beta, f, p,
                                         aux_loss, aux_coef, workspace, as_stream(stream)));
}

int moe_grouped_gate_up_train(const moe_shape* shape, const void* x_perm, const int32_t* sorted_token,
                              const void* x, const int32_t* offsets, const void* w_gate_up,
                              const void* ws_gate_up, void* gu, void* h, void* stream) {
  if (int r = check_train_shape(shape)) return r;
  if (shape->T == 0) return ok();
  OPT_PTR(x_perm);
  if (x_perm == nullptr) NEED_PTR(sorted_token);
  NEED_PTR(x);
  NEED_PTR(offsets);
  NEED_PTR(w_gate_up);
  if (shape->Fs > 0) NEED_PTR(ws_gate_up);
  NEED_PTR(gu);
  NEED_PTR(h);
  const moe_shape& s = *shape;
  using moe::bf16_t;
  hipError_t e = moe::launch_gate_up_pre_bf16(s, static_cast<const bf16_t*>(x_perm), sorted_token,
                                              static_cast<const bf16_t*>(x), offsets,
                                              static_cast<const bf16_t*>(w_gate_up),
                                              static_cast<const bf16_t*>(ws_gate_up),
                                              static_cast<bf16_t*>(gu), as_stream(stream));
  if (e == hipSuccess)
    e = moe::launch_swiglu_pre(s, static_cast<const bf16_t*>(gu), offsets, static_cast<bf16_t*>(h),
                               as_stream(stream));
  return launched(e);
}

int moe_combine_backward(const moe_shape* shape, const void* dout, const void* y_perm,
                         const int32_t* slot_of, const int32_t* topk_idx, const float* topk_w,
                         const float* logits, const float* aux_coef, void* dy_perm, float* dz,
                         void* dz_bf16, void* stream) {
  if (int r = check_train_shape(shape)) return r;
  if (shape->T == 0) return ok();
  NEED_PTR(dout);
  NEED_PTR(y_perm);
  NEED_PTR(slot_of);
  NEED_PTR(topk_idx);
  NEED_PTR(topk_w);
  NEED_PTR(logits);
  OPT_PTR(aux_coef);
  NEED_PTR(dy_perm);
  NEED_PTR(dz);
  NEED_PTR(dz_bf16);
  using moe::bf16_t;
  return launched(moe::launch_combine_bwd(*shape, static_cast<const bf16_t*>(dout),
                                          static_cast<const bf16_t*>(y_perm), slot_of, topk_idx, topk_w,
                                          logits, aux_coef, static_cast<bf16_t*>(dy_perm), dz,
                                          static_cast<bf16_t*>(dz_bf16), as_stream(stream)));
}

int moe_grouped_backward_h(const moe_shape* shape, const void* dy_perm, const void* dout,
                           const int32_t* offsets, const void* w_down_t, const void* ws_down_t,
                           const void* gu, void* dh, void* dgu, void* stream) {
  if (int r = check_train_shape(shape)) return r;
  if (shape->T == 0) return ok();
  NEED_PTR(dy_perm);
  NEED_PTR(offsets);
  NEED_PTR(w_down_t);
  if (shape->Fs > 0) {
    NEED_PTR(dout);
    NEED_PTR(ws_down_t);
  }
  NEED_PTR(gu);
  NEED_PTR(dh);
  NEED_PTR(dgu);
  const moe_shape& s = *shape;
  using moe::bf16_t;
  hipError_t e = moe::launch_dgrad_h_bf16(s, static_cast<const bf16_t*>(dy_perm),
                                          static_cast<const bf16_t*>(dout), offsets,
                                          static_cast<const bf16_t*>(w_down_t),
                                          static_cast<const bf16_t*>(ws_down_t), static_cast<bf16_t*>(dh),
                                          as_stream(stream));
  if (e == hipSuccess)
    e = moe::launch_swiglu_bwd(s, static_cast<const bf16_t*>(dh), static_cast<const bf16_t*>(gu), offsets,
                               static_cast<bf16_t*>(dgu), as_stream(stream));
  return launched(e);
}

int moe_grouped_backward_x(const moe_shape* shape, const void* dgu, const int32_t* offsets,
                           const void* w_gate_up_t, const void* ws_gate_up_t, const void* dz_bf16,
                           const void* w_router_t, const int32_t* slot_of, void* dx_perm, void* dx_shared,
                           void* dx_router, void* dx, void* stream) {
  if (int r = check_train_shape(shape)) return r;
  if (shape->T == 0) return ok();
  NEED_PTR(dgu);
  NEED_PTR(offsets);
  NEED_PTR(w_gate_up_t);
  if (shape->Fs > 0) {
    NEED_PTR(ws_gate_up_t);
    NEED_PTR(dx_shared);
  }
  NEED_PTR(dz_bf16);
  NEED_PTR(w_router_t);
  NEED_PTR(slot_of);
  NEED_PTR(dx_perm);
  NEED_PTR(dx_router);
  NEED_PTR(dx);
  const moe_shape& s = *shape;
  using moe::bf16_t;
  const hipStream_t st = as_stream(stream);
  bf16_t* dxs = s.Fs > 0 ? static_cast<bf16_t*>(dx_shared) : nullptr;
  hipError_t e = moe::launch_dgrad_x_bf16(s, static_cast<const bf16_t*>(dgu), offsets,
                                          static_cast<const bf16_t*>(w_gate_up_t),
                                          static_cast<const bf16_t*>(ws_gate_up_t),
                                          static_cast<bf16_t*>(dx_perm), dxs, st);
  if (e == hipSuccess)
    e = moe::launch_dense_bf16(s.T, 256, s.D, static_cast<const bf16_t*>(dz_bf16),
                               static_cast<const bf16_t*>(w_router_t), static_cast<bf16_t*>(dx_router), st);
  if (e == hipSuccess)
    e = moe::launch_dx_reduce(s, static_cast<const bf16_t*>(dx_perm), dxs,
                              static_cast<const bf16_t*>(dx_router), slot_of, static_cast<bf16_t*>(dx), st);
  return launched(e);
}

int moe_weight_grads(const moe_shape* shape, const void* x, const int32_t* sorted_token,
                     const void* x_perm, const int32_t* offsets, const void* dgu, const void* dy_perm,
                     const void* dout, const void* h, const void* dz_bf16, void* dw_gate_up, void* dw_down,
                     void* dws_gate_up, void* dws_down, float* dw_router, void* stream) {
  if (int r = check_train_shape(shape)) return r;
  const moe_shape& s = *shape;
  // with no tokens every gradient is zero and no input is read
  if (s.T > 0) {
    NEED_PTR(x);
    OPT_PTR(x_perm);
    if (x_perm == nullptr) NEED_PTR(sorted_token);
    NEED_PTR(offsets);
    NEED_PTR(dgu);
    NEED_PTR(dy_perm);
    NEED_PTR(h);
    if (s.Fs > 0) NEED_PTR(dout);
    if (dw_router) NEED_PTR(dz_bf16);
  }
  NEED_PTR(dw_gate_up);
  NEED_PTR(dw_down);
  if (s.Fs > 0) {
    NEED_PTR(dws_gate_up);
    NEED_PTR(dws_down);
  }
  OPT_PTR(dw_router);
  using moe::bf16_t;
  return launched(moe::launch_wgrad(
      s, static_cast<const bf16_t*>(x), sorted_token, static_cast<const bf16_t*>(x_perm),
      static_cast<const bf16_t*>(dgu), static_cast<const bf16_t*>(dy_perm), static_cast<const bf16_t*>(h),
      static_cast<const bf16_t*>(dout), static_cast<const bf16_t*>(dz_bf16), offsets,
      static_cast<bf16_t*>(dw_gate_up), static_cast<bf16_t*>(dw_down), static_cast<bf16_t*>(dws_gate_up),
      static_cast<bf16_t*>(dws_down), dw_router, as_stream(stream)));
}

int moe_bias_grad(const moe_shape* shape, const float* dz, float* dbias, void* workspace,
                  size_t workspace_bytes, void* stream) {
  if (int r = check_shape(shape)) return r;
  if (shape->T > 0) NEED_PTR(dz);
  NEED_PTR(dbias);
  if (int r = check_workspace(workspace, workspace_bytes, moe::train_workspace_bytes(*shape))) return r;
  return launched(moe::launch_colsum(*shape, dz, dbias, workspace, as_stream(stream)));
}

}  // extern "C"
