// Small helper kernels: fills, fp32 -> dtype conversion, and the
// deterministic reduction of the alignment losses.
//
// L_sparsity and L_commit have the same value, the mean of
// (h_full - h_sparse)^2 over all B*Hq*N*d elements of the layer; they differ
// only in which output their gradient moves (Sintesi Tecnica, section 2,
// 'Allineamento Bidirezionale').  The forward kernels leave one partial sum
// per row (or per tile); this kernel adds them in a fixed order in fp64.

#include "common.h"
#include "internal.h"

namespace ssa {

__global__ void k_zero_f32(float* __restrict__ p, int64_t n) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0.f;
}

void launch_zero_f32(float* p, int64_t n, hipStream_t s) {
  if (n <= 0) return;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  timing_begin(kKZero, s);
  hipLaunchKernelGGL(k_zero_f32, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, p, n);
  timing_end(kKZero, s);
}

template <typename T>
__global__ void k_convert(const float* __restrict__ src, T* __restrict__ dst, int64_t n) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
    dst[i] = from_f32<T>(src[i]);
}

void launch_convert(const float* src, void* dst, int dtype, int64_t n, hipStream_t s) {
  if (n <= 0) return;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  timing_begin(kKConvert, s);
  if (dtype == 1)
    hipLaunchKernelGGL(k_convert<bf16_t>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, src,
                       static_cast<bf16_t*>(dst), n);
  else
    hipLaunchKernelGGL(k_convert<float>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, src,
                       static_cast<float*>(dst), n);
  timing_end(kKConvert, s);
}

// Two levels, both in a fixed order (deterministic): workgroup w adds the
// contiguous chunk w of the row partials in fp64 (thread strides, then a
// tree), then one workgroup adds the kLossParts workgroup sums by a tree.
constexpr int kLossParts = 256;

__device__ __forceinline__ double block_sum_f64(double acc, double* buf) {
  buf[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if (static_cast<int>(threadIdx.x) < w) buf[threadIdx.x] += buf[threadIdx.x + w];
    __syncthreads();
  }
  return buf[0];
}

__global__ void __launch_bounds__(256) k_loss_partial(const float* __restrict__ part, int64_t n,
                                                      double* __restrict__ sums) {
  __shared__ double buf[256];
  const int64_t chunk = (n + kLossParts - 1) / kLossParts;
  const int64_t i0 = static_cast<int64_t>(blockIdx.x) * chunk;
  const int64_t i1 = i0 + chunk < n ? i0 + chunk : n;
  double acc = 0.0;
  for (int64_t i = i0 + threadIdx.x; i < i1; i += 256) acc += static_cast<double>(part[i]);
  const double t = block_sum_f64(acc, buf);
  if (threadIdx.x == 0) sums[blockIdx.x] = t;
}

__global__ void __launch_bounds__(256) k_loss_final(const double* __restrict__ sums, double inv_count,
                                                    float* __restrict__ losses) {
  __shared__ double buf[256];
  const double t = block_sum_f64(sums[threadIdx.x], buf);
  if (threadIdx.x == 0) {
    const float L = static_cast<float>(t * inv_count);
    losses[0] = L;   // L_sparsity
    losses[1] = L;   // L_commit
  }
}

// Per-head means of two per-row arrays: workgroup h adds rows h*N .. h*N+N-1
// of each in fp64 (fixed order), out[2h] and out[2h+1] = the sums / N.
__global__ void __launch_bounds__(256) k_head_means(const float* __restrict__ a, const float* __restrict__ b,
                                                    int N, float* __restrict__ out) {
  __shared__ double buf[256];
  const int64_t base = static_cast<int64_t>(blockIdx.x) * N;
  double sa = 0.0, sb = 0.0;
  for (int i = threadIdx.x; i < N; i += 256) {
    sa += static_cast<double>(a[base + i]);
    sb += static_cast<double>(b[base + i]);
  }
  const double ta = block_sum_f64(sa, buf);
  __syncthreads();                        // buf is reused
  const double tb = block_sum_f64(sb, buf);
  if (threadIdx.x == 0) {
    out[2 * static_cast<int64_t>(blockIdx.x)] = static_cast<float>(ta / N);
    out[2 * static_cast<int64_t>(blockIdx.x) + 1] = static_cast<float>(tb / N);
  }
}

void launch_head_means(const float* a, const float* b, int64_t n_heads, int N, float* out, hipStream_t s) {
  timing_begin(kKLossReduce, s);
  hipLaunchKernelGGL(k_head_means, dim3(static_cast<unsigned>(n_heads)), dim3(256), 0, s, a, b, N, out);
  timing_end(kKLossReduce, s);
}

size_t loss_scratch_bytes() { return kLossParts * sizeof(double); }

void launch_loss_reduce(const float* row_sq, int64_t n_rows, double inv_count, double* scratch, float* losses,
                        hipStream_t s) {
  timing_begin(kKLossReduce, s);
  hipLaunchKernelGGL(k_loss_partial, dim3(kLossParts), dim3(256), 0, s, row_sq, n_rows, scratch);
  hipLaunchKernelGGL(k_loss_final, dim3(1), dim3(256), 0, s, scratch, inv_count, losses);
  timing_end(kKLossReduce, s);
}

}  // namespace ssa
