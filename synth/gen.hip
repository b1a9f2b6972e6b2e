// Device twin of synth/__init__.py: fills HBM tensors with the same seeded,
// counter-based values the NumPy generator computes for the same indices.
// Input infrastructure only -- it holds none of the sparse-attention method.
//
// Value at flat index i of tensor `tid`:
//   h = SplitMix64(seed ^ (tid << 48) ^ i)   (Steele, Lea, Flood, OOPSLA 2014)
//   S = sum of the four 16-bit lanes of h;  x = float(S - 131070) * scale
// RMS rows: ss = sequential fp32 sum of squares of the row's bf16 values,
// inv = 1 / sqrt(ss / width + eps), value = bf16(x_bf16 * inv); division and
// square root are IEEE correctly rounded and nothing is contracted, so the
// bits equal the host generator's.
#include <hip/hip_runtime.h>
#include <stdint.h>

#pragma clang fp contract(off)

namespace {

__device__ __forceinline__ uint64_t splitmix64(uint64_t x) {
    uint64_t z = x + 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

__device__ __forceinline__ float draw(uint64_t base, uint64_t i, float scale) {
    const uint64_t h = splitmix64(i ^ base);
    const int32_t s = (int32_t)((h & 0xFFFF) + ((h >> 16) & 0xFFFF) + ((h >> 32) & 0xFFFF) + (h >> 48));
    return (float)(s - 131070) * scale;
}

__device__ __forceinline__ uint16_t to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__global__ void fill_bf16_kernel(uint16_t* out, uint64_t n, uint64_t base, uint64_t idx0, float scale) {
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (uint64_t)gridDim.x * blockDim.x)
        out[i] = to_bf16(draw(base, idx0 + i, scale));
}

__global__ void fill_f32_kernel(float* out, uint64_t n, uint64_t base, uint64_t idx0, float scale) {
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (uint64_t)gridDim.x * blockDim.x)
        out[i] = draw(base, idx0 + i, scale);
}

__global__ void fill_rms_rows_kernel(uint16_t* out, uint64_t n_rows, int width, uint64_t base,
                                     uint64_t row0, float scale, float eps) {
    for (uint64_t r = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; r < n_rows;
         r += (uint64_t)gridDim.x * blockDim.x) {
        const uint64_t i0 = (row0 + r) * (uint64_t)width;
        float ss = 0.0f;
        for (int j = 0; j < width; ++j) {
            const float x = __uint_as_float((uint32_t)to_bf16(draw(base, i0 + j, scale)) << 16);
            ss = ss + x * x;
        }
        const float mean = ss / (float)width;
        const float inv = 1.0f / sqrtf(mean + eps);
        uint16_t* o = out + r * (uint64_t)width;
        for (int j = 0; j < width; ++j) {
            const float x = __uint_as_float((uint32_t)to_bf16(draw(base, i0 + j, scale)) << 16);
            o[j] = to_bf16(x * inv);
        }
    }
}

// correlated rows: x = sum over j = 0 .. window-1 (in that order) of the draw
// at ((row + window - 1 - j) * width + e), then x * c (c = fp32(1/sqrt(window)))
__global__ void fill_corr_kernel(void* out, int bf16_out, uint64_t n_rows, int width, int window,
                                 uint64_t base, uint64_t row0, float scale, float c) {
    const uint64_t n = n_rows * (uint64_t)width;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (uint64_t)gridDim.x * blockDim.x) {
        const uint64_t r = row0 + i / (uint64_t)width;
        const uint64_t e = i % (uint64_t)width;
        float acc = 0.0f;
        for (int j = 0; j < window; ++j)
            acc = acc + draw(base, (r + (uint64_t)(window - 1 - j)) * (uint64_t)width + e, scale);
        const float x = acc * c;
        if (bf16_out)
            ((uint16_t*)out)[i] = to_bf16(x);
        else
            ((float*)out)[i] = x;
    }
}

unsigned grid_for(uint64_t n, unsigned block) {
    uint64_t g = (n + block - 1) / block;
    return (unsigned)(g > 65536 * 4 ? 65536 * 4 : (g == 0 ? 1 : g));
}

uint64_t stream_base(uint64_t seed, uint32_t tid) { return seed ^ ((uint64_t)tid << 48); }

}  // namespace

extern "C" {

int synth_fill_bf16(void* out, uint64_t n, uint64_t seed, uint32_t tid, uint64_t idx0, float scale,
                    void* stream) {
    if (n == 0) return 0;
    hipLaunchKernelGGL(fill_bf16_kernel, dim3(grid_for(n, 256)), dim3(256), 0, (hipStream_t)stream,
                       (uint16_t*)out, n, stream_base(seed, tid), idx0, scale);
    return (int)hipGetLastError();
}

int synth_fill_f32(float* out, uint64_t n, uint64_t seed, uint32_t tid, uint64_t idx0, float scale,
                   void* stream) {
    if (n == 0) return 0;
    hipLaunchKernelGGL(fill_f32_kernel, dim3(grid_for(n, 256)), dim3(256), 0, (hipStream_t)stream,
                       out, n, stream_base(seed, tid), idx0, scale);
    return (int)hipGetLastError();
}

int synth_fill_rms_rows_bf16(void* out, uint64_t n_rows, int32_t width, uint64_t seed, uint32_t tid,
                             uint64_t row0, float scale, float eps, void* stream) {
    if (n_rows == 0) return 0;
    hipLaunchKernelGGL(fill_rms_rows_kernel, dim3(grid_for(n_rows, 128)), dim3(128), 0,
                       (hipStream_t)stream, (uint16_t*)out, n_rows, (int)width,
                       stream_base(seed, tid), row0, scale, eps);
    return (int)hipGetLastError();
}

int synth_fill_corr(void* out, int32_t bf16_out, uint64_t n_rows, int32_t width, int32_t window,
                    uint64_t seed, uint32_t tid, uint64_t row0, float scale, float c, void* stream) {
    if (n_rows == 0) return 0;
    if (width <= 0 || window <= 0) return (int)hipErrorInvalidValue;
    const uint64_t n = n_rows * (uint64_t)width;
    hipLaunchKernelGGL(fill_corr_kernel, dim3(grid_for(n, 256)), dim3(256), 0, (hipStream_t)stream, out,
                       (int)bf16_out, n_rows, (int)width, (int)window, stream_base(seed, tid), row0, scale, c);
    return (int)hipGetLastError();
}

}  // extern "C"
