// Reconstruction loss of a quantized matrix under an arbitrary Hessian,
//   loss = sum_r (Wq_r - W_r) H (Wq_r - W_r)^T ,
// with column k of Wq on grid gidx[k] (or k / group when no g_idx is given),
// the per-layer term of the objective in the CLHA summary, section 2.1 (with
// H = H_comb it is the combined objective; with H = H_a or H_b it is the error
// a shared weight leaves on one layer's calibration data).
//
// Each workgroup forms a 64x64 tile of Y = Delta H on the fp32 matrix cores
// (v_mfma_f32_32x32x2f32), Delta dequantized on the fly from codes, scales and
// zero points, then reduces sum Y .* Delta over its tile into one fp64 partial;
// a second kernel adds the partials in a fixed order.
#include "kernels.h"

#include <mutex>

namespace clha {

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float delta_at(const void* W, int dtype, const uint8_t* codes,
                                          const float* scales, const uint8_t* zeros, const int* gidx,
                                          int cols, int group, int r, int k) {
  const int64_t gi = (int64_t)r * (cols / group) + (gidx ? gidx[k] : k / group);
  const float wq = scales[gi] * ((float)codes[(int64_t)r * cols + k] - (float)zeros[gi]);
  float w;
  if (dtype == 1) w = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(W)[(int64_t)r * cols + k] << 16);
  else w = reinterpret_cast<const float*>(W)[(int64_t)r * cols + k];
  return wq - w;
}

__global__ __launch_bounds__(256) void loss_tile_kernel(int rows, int cols, int group, const void* W,
                                                        int dtype, const uint8_t* __restrict__ codes,
                                                        const float* __restrict__ scales,
                                                        const uint8_t* __restrict__ zeros,
                                                        const float* __restrict__ H,
                                                        const int* __restrict__ gidx,
                                                        double* __restrict__ partials) {
  __shared__ float Ds[64][65];   // Delta chunk, [k][row]
  __shared__ float Hs[64][65];   // H chunk, [k][col]
  __shared__ double red[256];
  const int j0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, kh = lane >> 5;
  const int arow = wm * 32 + (lane & 31), bcol = wn * 32 + (lane & 31);
  f32x16 acc = f32x16{};
  for (int k0 = 0; k0 < cols; k0 += 64) {
    __syncthreads();
    for (int idx = tid; idx < 64 * 64; idx += 256) {
      const int a = idx >> 6, b = idx & 63;     // a: row (Delta) / k (H), b: k (Delta) / col (H)
      Ds[b][a] = (r0 + a < rows) ? delta_at(W, dtype, codes, scales, zeros, gidx, cols, group, r0 + a, k0 + b) : 0.0f;
      Hs[a][b] = H[(int64_t)(k0 + a) * cols + j0 + b];
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < 64; kk += 2) {
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(Ds[kk + kh][arow], Hs[kk + kh][bcol], acc, 0, 0, 0);
    }
  }
  double part = 0.0;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = r0 + wm * 32 + 8 * (r >> 2) + 4 * kh + (r & 3);
    if (row < rows)
      part += (double)acc[r] *
              (double)delta_at(W, dtype, codes, scales, zeros, gidx, cols, group, row, j0 + bcol);
  }
  red[tid] = part;
  __syncthreads();
  for (int st = 128; st > 0; st >>= 1) {
    if (tid < st) red[tid] += red[tid + st];
    __syncthreads();
  }
  if (tid == 0) partials[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] = red[0];
}

__global__ void loss_finish_kernel(const double* __restrict__ partials, int64_t n, float* out) {
  if (threadIdx.x != 0) return;
  double s = 0.0;
  for (int64_t i = 0; i < n; ++i) s += partials[i];
  out[0] = (float)s;
}

int64_t loss_partial_count(int rows, int cols) {
  return (int64_t)(cols / 64) * ((rows + 63) / 64);
}

// Scratch of the allocation-free loss entry point: the fp64 tile partials live
// in this file-scope device array instead of a caller workspace.  Each device
// holds its own copy; its address is looked up once per device (with that
// device current) by loss_scratch_init, and only that address is ever passed to
// kernels: in host code the array's name is not a device address.
static __device__ __align__(256) double scratch[kLossScratchPartials];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
double* g_scratch[kMaxScratchDevices] = {};
}  // namespace

bool loss_scratch_init(int device) {
  if (device < 0 || device >= kMaxScratchDevices) return false;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch[device]) return true;
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return false;
  g_scratch[device] = static_cast<double*>(ptr);
  return true;
}

double* loss_scratch(int device) {
  if (device < 0 || device >= kMaxScratchDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  return g_scratch[device];
}

void launch_loss(int rows, int cols, int group, const void* W, int dtype, const uint8_t* codes,
                 const float* scales, const uint8_t* zeros, const float* H, const int* gidx,
                 float* partials, float* loss_out, hipStream_t s) {
  double* part = reinterpret_cast<double*>(partials);
  hipLaunchKernelGGL(loss_tile_kernel, dim3(cols / 64, (rows + 63) / 64), dim3(256), 0, s, rows,
                     cols, group, W, dtype, codes, scales, zeros, H, gidx, part);
  hipLaunchKernelGGL(loss_finish_kernel, dim3(1), dim3(64), 0, s, part,
                     loss_partial_count(rows, cols), loss_out);
}

}  // namespace clha
