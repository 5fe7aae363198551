// layer_ops.hip -- the elementwise and row-reduction steps of the decoder block
// around the attention path (RMSNorm, rotary positions, SwiGLU), forward and
// backward, fused into one kernel each.
//
// Not steps of the attention method itself: the OOMB page trains Qwen2.5-7B,
// whose decoder block puts RMSNorm before the attention and the MLP, rotary
// positions on q and k, and a SwiGLU MLP around the paged attention.  These
// kernels let that block run chunk by chunk without a chain of small framework
// kernels per step.  All accumulation is fp32; bf16 values are rounded once
// (RNE) when written.
#include "common.h"
#include "oomb.h"

namespace oomb {

constexpr int kRowThreads = 256;
constexpr int kRowMaxVec = 8;  // float4 chunks a thread keeps: hidden sizes up to 256 * 4 * 8 = 8192

typedef __attribute__((ext_vector_type(4))) __bf16 bf16v4;

__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  const int w = threadIdx.x >> 6;
  __syncthreads();  // red may still be read by an earlier call
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kRowThreads / 64; ++i) s += red[i];
  return s;
}

// h = x * rstd * gain, rstd = 1 / sqrt(mean(x^2) + eps); one workgroup per row.
__global__ __launch_bounds__(kRowThreads) void rmsnorm_fwd_kernel(const float* __restrict__ x,
                                                                  const __bf16* __restrict__ gain, int H, float eps,
                                                                  __bf16* __restrict__ h, float* __restrict__ rstd) {
  __shared__ float red[kRowThreads / 64];
  const int64_t row = blockIdx.x;
  const f32x4* xr = reinterpret_cast<const f32x4*>(x + row * H);
  const int nv = H / 4;
  f32x4 v[kRowMaxVec];
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < kRowMaxVec; ++k) {
    const int i = threadIdx.x + k * kRowThreads;
    v[k] = i < nv ? xr[i] : f32x4{0.f, 0.f, 0.f, 0.f};
    ss += v[k][0] * v[k][0] + v[k][1] * v[k][1] + v[k][2] * v[k][2] + v[k][3] * v[k][3];
  }
  const float r = rsqrtf(block_sum(ss, red) / H + eps);
  const bf16v4* gr = reinterpret_cast<const bf16v4*>(gain);
  bf16v4* hr = reinterpret_cast<bf16v4*>(h + row * H);
#pragma unroll
  for (int k = 0; k < kRowMaxVec; ++k) {
    const int i = threadIdx.x + k * kRowThreads;
    if (i < nv) {
      const bf16v4 g = gr[i];
      bf16v4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = (__bf16)(v[k][e] * r * (float)g[e]);
      hr[i] = o;
    }
  }
  if (threadIdx.x == 0) rstd[row] = r;
}

// dx = r * g * dh - x * r^3 * mean(g * dh * x)  (+ dres when given)
__global__ __launch_bounds__(kRowThreads) void rmsnorm_bwd_kernel(const float* __restrict__ x,
                                                                  const __bf16* __restrict__ gain,
                                                                  const float* __restrict__ rstd,
                                                                  const __bf16* __restrict__ dh,
                                                                  const float* __restrict__ dres, int H,
                                                                  float* __restrict__ dx) {
  __shared__ float red[kRowThreads / 64];
  const int64_t row = blockIdx.x;
  const int nv = H / 4;
  const f32x4* xr = reinterpret_cast<const f32x4*>(x + row * H);
  const bf16v4* dr = reinterpret_cast<const bf16v4*>(dh + row * H);
  const bf16v4* gr = reinterpret_cast<const bf16v4*>(gain);
  f32x4 xv[kRowMaxVec], gd[kRowMaxVec];
  float dot = 0.f;
#pragma unroll
  for (int k = 0; k < kRowMaxVec; ++k) {
    const int i = threadIdx.x + k * kRowThreads;
    xv[k] = gd[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (i < nv) {
      xv[k] = xr[i];
      const bf16v4 d = dr[i], g = gr[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) gd[k][e] = (float)g[e] * (float)d[e];
    }
    dot += gd[k][0] * xv[k][0] + gd[k][1] * xv[k][1] + gd[k][2] * xv[k][2] + gd[k][3] * xv[k][3];
  }
  const float r = rstd[row];
  const float c = block_sum(dot, red) / H * r * r * r;
  f32x4* out = reinterpret_cast<f32x4*>(dx + row * H);
  const f32x4* res = dres ? reinterpret_cast<const f32x4*>(dres + row * H) : nullptr;
#pragma unroll
  for (int k = 0; k < kRowMaxVec; ++k) {
    const int i = threadIdx.x + k * kRowThreads;
    if (i < nv) {
      f32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = r * gd[k][e] - xv[k][e] * c;
      if (res) o += res[i];
      out[i] = o;
    }
  }
}

// partial[s][j] = sum over rows r of segment s of dh[r][j] * x[r][j] * rstd[r]
// (the gain gradient is the sum of the partials over s); a thread per column
// of a segment.
__global__ __launch_bounds__(256) void rmsnorm_gain_grad_kernel(const float* __restrict__ x,
                                                                const float* __restrict__ rstd,
                                                                const __bf16* __restrict__ dh, int rows, int H,
                                                                int rows_per_seg, float* __restrict__ partial) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  const int s = blockIdx.y;
  if (j >= H) return;
  const int r0 = s * rows_per_seg, r1 = min(rows, r0 + rows_per_seg);
  float acc = 0.f;
  for (int r = r0; r < r1; ++r) acc += (float)dh[(int64_t)r * H + j] * x[(int64_t)r * H + j] * rstd[r];
  partial[(int64_t)s * H + j] = acc;
}

// Rotate-half rotary positions: for token r (position pos0 + r), pair
// (j, j + D/2) of every head turns by the angle whose cosine and sine are
// cos[pos][j], sin[pos][j]; inverse turns the other way (the transpose, for
// gradients).  in: fp32 or bf16 [rows][heads][D]; out: bf16.
template <typename Tin>
__global__ __launch_bounds__(256) void rotary_kernel(const Tin* __restrict__ in, __bf16* __restrict__ out,
                                                     const float* __restrict__ cosv, const float* __restrict__ sinv,
                                                     int rows, int heads, int half, int pos0, float sign) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (row, head, j < half)
  if (i >= (int64_t)rows * heads * half) return;
  const int j = (int)(i % half);
  const int64_t rh = i / half;
  const int r = (int)(rh / heads);
  const int64_t base = rh * 2 * half;
  const float a = (float)in[base + j], b = (float)in[base + half + j];
  const float c = cosv[(int64_t)(pos0 + r) * half + j], s = sign * sinv[(int64_t)(pos0 + r) * half + j];
  out[base + j] = (__bf16)(a * c - b * s);
  out[base + half + j] = (__bf16)(b * c + a * s);
}

// m = silu(g) * u
__global__ __launch_bounds__(256) void swiglu_fwd_kernel(const __bf16* __restrict__ g, const __bf16* __restrict__ u,
                                                         __bf16* __restrict__ m, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const bf16v4 gv = reinterpret_cast<const bf16v4*>(g)[i], uv = reinterpret_cast<const bf16v4*>(u)[i];
  bf16v4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float x = (float)gv[e];
    o[e] = (__bf16)(x / (1.f + __expf(-x)) * (float)uv[e]);
  }
  reinterpret_cast<bf16v4*>(m)[i] = o;
}

// dg = dm * u * silu'(g), du = dm * silu(g); silu'(x) = s + x s (1 - s), s = sigmoid(x)
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const __bf16* __restrict__ g, const __bf16* __restrict__ u,
                                                         const __bf16* __restrict__ dm, __bf16* __restrict__ dg,
                                                         __bf16* __restrict__ du, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const bf16v4 gv = reinterpret_cast<const bf16v4*>(g)[i], uv = reinterpret_cast<const bf16v4*>(u)[i];
  const bf16v4 dv = reinterpret_cast<const bf16v4*>(dm)[i];
  bf16v4 og, ou;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float x = (float)gv[e], d = (float)dv[e];
    const float s = 1.f / (1.f + __expf(-x));
    og[e] = (__bf16)(d * (float)uv[e] * (s + x * s * (1.f - s)));
    ou[e] = (__bf16)(d * x * s);
  }
  reinterpret_cast<bf16v4*>(dg)[i] = og;
  reinterpret_cast<bf16v4*>(du)[i] = ou;
}

}  // namespace oomb

// ---------------------------------------------------------------------------
// C ABI (declared in include/oomb.h).  Host checks run before any HIP call.
// ---------------------------------------------------------------------------
#define OOMB_API extern "C" __attribute__((visibility("default")))

namespace {
bool bad16(const void* p) { return ((uintptr_t)p & 15u) != 0; }
bool bad8(const void* p) { return ((uintptr_t)p & 7u) != 0; }
int launch_status() { return hipGetLastError() == hipSuccess ? OOMB_OK : OOMB_ERR_LAUNCH; }
}  // namespace

OOMB_API int oomb_rmsnorm_fwd(const float* x, const void* gain, int32_t rows, int32_t hidden, float eps, void* h,
                              float* rstd, void* stream) {
  if (!x || !gain || !h || !rstd) return OOMB_ERR_NULL_PTR;
  if (rows < 0 || hidden <= 0 || hidden % 4 || hidden > oomb::kRowThreads * 4 * oomb::kRowMaxVec || !(eps >= 0.f))
    return OOMB_ERR_BAD_SHAPE;
  if (bad16(x) || bad8(gain) || bad8(h)) return OOMB_ERR_MISALIGNED;
  if (rows == 0) return OOMB_OK;
  (void)hipGetLastError();
  hipLaunchKernelGGL(oomb::rmsnorm_fwd_kernel, dim3(rows), dim3(oomb::kRowThreads), 0, (hipStream_t)stream, x,
                     (const __bf16*)gain, hidden, eps, (__bf16*)h, rstd);
  return launch_status();
}

OOMB_API int oomb_rmsnorm_bwd(const float* x, const void* gain, const float* rstd, const void* dh, const float* dres,
                              int32_t rows, int32_t hidden, float* dx, void* stream) {
  if (!x || !gain || !rstd || !dh || !dx) return OOMB_ERR_NULL_PTR;
  if (rows < 0 || hidden <= 0 || hidden % 4 || hidden > oomb::kRowThreads * 4 * oomb::kRowMaxVec) return OOMB_ERR_BAD_SHAPE;
  if (bad16(x) || bad8(gain) || bad8(dh) || bad16(dx) || (dres && bad16(dres))) return OOMB_ERR_MISALIGNED;
  if (rows == 0) return OOMB_OK;
  (void)hipGetLastError();
  hipLaunchKernelGGL(oomb::rmsnorm_bwd_kernel, dim3(rows), dim3(oomb::kRowThreads), 0, (hipStream_t)stream, x,
                     (const __bf16*)gain, rstd, (const __bf16*)dh, dres, hidden, dx);
  return launch_status();
}

OOMB_API int oomb_rmsnorm_gain_grad(const float* x, const float* rstd, const void* dh, int32_t rows, int32_t hidden,
                                    int32_t segments, float* partial, void* stream) {
  if (!x || !rstd || !dh || !partial) return OOMB_ERR_NULL_PTR;
  if (rows < 0 || hidden <= 0 || segments < 1 || segments > 65535) return OOMB_ERR_BAD_SHAPE;
  (void)hipGetLastError();
  const int per = rows > 0 ? (rows + segments - 1) / segments : 1;
  hipLaunchKernelGGL(oomb::rmsnorm_gain_grad_kernel, dim3((hidden + 255) / 256, segments), dim3(256), 0,
                     (hipStream_t)stream, x, rstd, (const __bf16*)dh, rows, hidden, per, partial);
  return launch_status();
}

OOMB_API int oomb_rotary(const void* in, int32_t in_dtype, void* out, const float* cos_table, const float* sin_table,
                         int32_t rows, int32_t heads, int32_t head_dim, int32_t first_position, int32_t inverse,
                         void* stream) {
  if (!in || !out || !cos_table || !sin_table) return OOMB_ERR_NULL_PTR;
  if (rows < 0 || heads <= 0 || head_dim <= 0 || head_dim % 2 || first_position < 0) return OOMB_ERR_BAD_SHAPE;
  if (in_dtype != 0 && in_dtype != 1) return OOMB_ERR_BAD_DTYPE;
  if (rows == 0) return OOMB_OK;
  (void)hipGetLastError();
  const int half = head_dim / 2;
  const int64_t n = (int64_t)rows * heads * half;
  const dim3 grid((unsigned)((n + 255) / 256));
  const float sign = inverse ? -1.f : 1.f;
  if (in_dtype == 0)
    hipLaunchKernelGGL(oomb::rotary_kernel<float>, grid, dim3(256), 0, (hipStream_t)stream, (const float*)in,
                       (__bf16*)out, cos_table, sin_table, rows, heads, half, first_position, sign);
  else
    hipLaunchKernelGGL(oomb::rotary_kernel<__bf16>, grid, dim3(256), 0, (hipStream_t)stream, (const __bf16*)in,
                       (__bf16*)out, cos_table, sin_table, rows, heads, half, first_position, sign);
  return launch_status();
}

OOMB_API int oomb_swiglu_fwd(const void* gate, const void* up, void* out, int64_t n, void* stream) {
  if (!gate || !up || !out) return OOMB_ERR_NULL_PTR;
  if (n < 0 || n % 4) return OOMB_ERR_BAD_SHAPE;
  if (bad8(gate) || bad8(up) || bad8(out)) return OOMB_ERR_MISALIGNED;
  if (n == 0) return OOMB_OK;
  (void)hipGetLastError();
  const int64_t n4 = n / 4;
  hipLaunchKernelGGL(oomb::swiglu_fwd_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, (hipStream_t)stream,
                     (const __bf16*)gate, (const __bf16*)up, (__bf16*)out, n4);
  return launch_status();
}

OOMB_API int oomb_swiglu_bwd(const void* gate, const void* up, const void* dout, void* dgate, void* dup, int64_t n,
                             void* stream) {
  if (!gate || !up || !dout || !dgate || !dup) return OOMB_ERR_NULL_PTR;
  if (n < 0 || n % 4) return OOMB_ERR_BAD_SHAPE;
  if (bad8(gate) || bad8(up) || bad8(dout) || bad8(dgate) || bad8(dup)) return OOMB_ERR_MISALIGNED;
  if (n == 0) return OOMB_OK;
  (void)hipGetLastError();
  const int64_t n4 = n / 4;
  hipLaunchKernelGGL(oomb::swiglu_bwd_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, (hipStream_t)stream,
                     (const __bf16*)gate, (const __bf16*)up, (const __bf16*)dout, (__bf16*)dgate, (__bf16*)dup, n4);
  return launch_status();
}
