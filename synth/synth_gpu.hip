// synth_gpu.hip -- GPU side of the seeded synthetic-input generator.
//
// Shared input generator for tests and benchmark (it holds none of the
// optimizer step's arithmetic). It is the same function of (seed, stream,
// element index) as synth_host.c: Philox4x32-10 (Salmon et al., SC 2011) on
// counter {lo32(i), hi32(i), 0, 0} and key {seed, stream}; the eight 16-bit
// halves summed (Irwin-Hall of 8); z = (2*S - 8*65535) * C in binary64;
// f = (float)(z * std) (or |z| * std); bf16 codes are the upper 16 bits of f.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint32_t kM0 = 0xD2511F53u;
constexpr uint32_t kM1 = 0xCD9E8D57u;
constexpr uint32_t kW0 = 0x9E3779B9u;
constexpr uint32_t kW1 = 0xBB67AE85u;
constexpr double kIrwinHallC = 0x1.3988e1412ed76p-17;

__device__ __forceinline__ double gen_z(uint64_t i, uint32_t seed, uint32_t stream)
{
    uint32_t c0 = static_cast<uint32_t>(i), c1 = static_cast<uint32_t>(i >> 32), c2 = 0u, c3 = 0u;
    uint32_t k0 = seed, k1 = stream;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r > 0) { k0 += kW0; k1 += kW1; }
        const uint32_t lo0 = kM0 * c0, hi0 = __umulhi(kM0, c0);
        const uint32_t lo1 = kM1 * c2, hi1 = __umulhi(kM1, c2);
        const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
        c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
    }
    const int32_t s = static_cast<int32_t>((c0 & 0xFFFFu) + (c0 >> 16) + (c1 & 0xFFFFu) + (c1 >> 16) +
                                           (c2 & 0xFFFFu) + (c2 >> 16) + (c3 & 0xFFFFu) + (c3 >> 16));
    const int32_t d = 2 * s - 8 * 65535;
    return __dmul_rn(static_cast<double>(d), kIrwinHallC);
}

__global__ void fill_f32_kernel(float* __restrict__ out, int64_t n, int64_t start, uint32_t seed, uint32_t stream,
                                double stdev, int32_t absval)
{
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
        double z = gen_z(static_cast<uint64_t>(start + i), seed, stream);
        if (absval) z = fabs(z);
        out[i] = __double2float_rn(__dmul_rn(z, stdev));
    }
}

__global__ void fill_bf16_kernel(uint16_t* __restrict__ out, int64_t n, int64_t start, uint32_t seed,
                                 uint32_t stream, double stdev)
{
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
        const double z = gen_z(static_cast<uint64_t>(start + i), seed, stream);
        const float f = __double2float_rn(__dmul_rn(z, stdev));
        out[i] = static_cast<uint16_t>(__float_as_uint(f) >> 16);
    }
}

unsigned grid_for(int64_t n)
{
    const int64_t blocks = (n + 255) / 256;
    return static_cast<unsigned>(blocks < 8192 ? (blocks > 0 ? blocks : 1) : 8192);
}

}  // namespace

extern "C" int synth_gpu_fill_f32(float* out, int64_t n, int64_t start, uint32_t seed, uint32_t stream, double stdev,
                                  int32_t absval, hipStream_t s)
{
    if (n <= 0) return 0;
    if (!out) return 1;
    fill_f32_kernel<<<grid_for(n), 256, 0, s>>>(out, n, start, seed, stream, stdev, absval);
    return static_cast<int>(hipGetLastError());
}

extern "C" int synth_gpu_fill_bf16(void* out, int64_t n, int64_t start, uint32_t seed, uint32_t stream, double stdev,
                                   hipStream_t s)
{
    if (n <= 0) return 0;
    if (!out) return 1;
    fill_bf16_kernel<<<grid_for(n), 256, 0, s>>>(static_cast<uint16_t*>(out), n, start, seed, stream, stdev);
    return static_cast<int>(hipGetLastError());
}
