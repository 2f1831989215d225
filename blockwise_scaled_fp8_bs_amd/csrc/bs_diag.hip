// Exhaustive device self-checks of the quantizers' arithmetic (bs_device.h).
#include "bs_device.h"
#include "bs_kernels.h"

namespace bs {

namespace {

constexpr uint32_t kBits464 = 0x43E80000u;  // 464.0f

// Census of the hot-path encode step (no clamp) over all |y| <= 464, both signs.
__global__ __launch_bounds__(256) void census_kernel(uint32_t* min_bits, uint32_t* max_bits,
                                                     unsigned long long* counts) {
    __shared__ uint32_t s_min[256], s_max[256];
    __shared__ unsigned long long s_cnt[256];
    for (int i = threadIdx.x; i < 256; i += blockDim.x) {
        s_min[i] = 0xffffffffu;
        s_max[i] = 0u;
        s_cnt[i] = 0ull;
    }
    __syncthreads();
    const uint64_t total = (uint64_t)kBits464 + 1;  // magnitudes 0 .. 464 inclusive
    const uint64_t per = (total + gridDim.x - 1) / gridDim.x;
    const uint64_t b0 = (uint64_t)blockIdx.x * per;
    const uint64_t b1 = b0 + per < total ? b0 + per : total;
    // Runs of equal codes are accumulated per thread before touching LDS.
    for (int sign = 0; sign < 2; ++sign) {
        uint32_t run_code = 0xffffffffu, run_lo = 0, run_hi = 0;
        unsigned long long run_n = 0;
        for (uint64_t i = b0 + threadIdx.x; i < b1; i += blockDim.x) {
            const uint32_t u = (uint32_t)i;
            const float y = __uint_as_float(u | (sign ? 0x80000000u : 0u));
            const uint32_t c = encode4(y, 0.f, 0.f, 0.f) & 0xffu;
            if (c != run_code) {
                if (run_n) {
                    atomicMin(&s_min[run_code], run_lo);
                    atomicMax(&s_max[run_code], run_hi);
                    atomicAdd(&s_cnt[run_code], run_n);
                }
                run_code = c;
                run_lo = u;
                run_n = 0;
            }
            run_hi = u;
            ++run_n;
        }
        if (run_n) {
            atomicMin(&s_min[run_code], run_lo);
            atomicMax(&s_max[run_code], run_hi);
            atomicAdd(&s_cnt[run_code], run_n);
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < 256; i += blockDim.x) {
        if (s_cnt[i]) {
            atomicMin(&min_bits[i], s_min[i]);
            atomicMax(&max_bits[i], s_max[i]);
            atomicAdd(&counts[i], s_cnt[i]);
        }
    }
}

__global__ void census_init(uint32_t* min_bits, uint32_t* max_bits, unsigned long long* counts) {
    const int i = threadIdx.x;
    min_bits[i] = 0xffffffffu;
    max_bits[i] = 0u;
    counts[i] = 0ull;
}

// One workgroup per amax candidate: every positive finite bf16 (bits
// 0x0001 .. 0x7F7F) plus amax = 0, which takes the EPS floor.  Every finite
// bf16 x with |x| <= max(amax, EPS) is divided by the block scale with the
// quantizers' routine and with the IEEE division; the codes of the
// routine (encode4, no clamp) are compared with the definition's codes
// (IEEE quotient, clamp, round).
// result[0] pairs checked, [1] scale mismatches, [2] e4m3 code mismatches,
// [3] quotient mismatches with |x/s| >= 2^-10, [4] quotient mismatches with
// |x/s| < 2^-10 (these encode to a signed zero either way; informational).
__global__ __launch_bounds__(256) void division_kernel(unsigned long long* result) {
    const uint32_t amax_bits = blockIdx.x;  // 0 .. 0x7F7F
    const float amax = __uint_as_float(amax_bits << 16);
    const Scale sc = block_scale(amax);
    const float s_ieee = fmaxf(amax, kEps) / kE4m3Max;
    unsigned long long c[5] = {0, 0, 0, 0, 0};
    if (threadIdx.x == 0 && __float_as_uint(sc.s) != __float_as_uint(s_ieee)) ++c[1];
    const float lim = fmaxf(amax, kEps);
    for (uint32_t xb = threadIdx.x; xb <= 0x7F7Fu; xb += blockDim.x) {
        const float xp = __uint_as_float(xb << 16);
        if (xp > lim) continue;
#pragma unroll
        for (int sg = 0; sg < 2; ++sg) {
            const float x = sg ? -xp : xp;
            const float y = div_by_scale(x, sc);
            const float y_ieee = x / s_ieee;
            ++c[0];
            if ((encode4(y, 0.f, 0.f, 0.f) & 0xffu) != encode_clamped(y_ieee)) ++c[2];
            if (__float_as_uint(y) != __float_as_uint(y_ieee)) {
                if (fabsf(y_ieee) >= 0.0009765625f) ++c[3];
                else ++c[4];
            }
        }
    }
#pragma unroll
    for (int k = 0; k < 5; ++k) {
        unsigned long long v = c[k];
        for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
        if ((threadIdx.x & 63) == 0 && v) atomicAdd(&result[k], v);
    }
}

__global__ void division_init(unsigned long long* result) {
    if (threadIdx.x < 5) result[threadIdx.x] = 0ull;
}

}  // namespace

hipError_t launch_diag_e4m3_census(uint32_t* min_bits, uint32_t* max_bits, unsigned long long* counts,
                                   hipStream_t stream) {
    hipLaunchKernelGGL(census_init, dim3(1), dim3(256), 0, stream, min_bits, max_bits, counts);
    hipLaunchKernelGGL(census_kernel, dim3(8192), dim3(256), 0, stream, min_bits, max_bits, counts);
    return hipGetLastError();
}

hipError_t launch_diag_division(unsigned long long* result, hipStream_t stream) {
    hipLaunchKernelGGL(division_init, dim3(1), dim3(64), 0, stream, result);
    hipLaunchKernelGGL(division_kernel, dim3(0x7F80), dim3(256), 0, stream, result);
    return hipGetLastError();
}

// Streaming reference for the HBM-bound kernels: reads n_read bytes of src
// and writes n_write >= n_read bytes of dst with the quantizers' access
// pattern (16-byte buffer loads and stores per lane, one workgroup of 256
// threads per 32 KiB of input, coalesced), so that its rate is the practical
// ceiling of a pass that moves the same bytes.  Written: the read bytes XOR 1
// (nothing folds away), then the n_write - n_read remaining bytes, spread
// evenly over the workgroups.  Both sizes are multiples of 16.
namespace {
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t stream_rsrc(const void* base, int64_t bytes) {
    const int32_t n = bytes > 0x7fffffff ? 0x7fffffff : (bytes < 0 ? 0 : (int32_t)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

constexpr int64_t kStreamChunk = 256 * 16 * 8;  // input bytes per workgroup

__global__ __launch_bounds__(256) void stream_kernel(const uint8_t* src, int64_t n_read, uint8_t* dst,
                                                     int64_t n_write) {
    const int64_t base = (int64_t)blockIdx.x * kStreamChunk;
    const int voff = threadIdx.x * 16;
    const __amdgpu_buffer_rsrc_t rs = stream_rsrc(src + base, n_read - base);
    const __amdgpu_buffer_rsrc_t rd = stream_rsrc(dst + base, n_read - base);
    u32x4_t v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
        v[k] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, k * 4096, 0));
#pragma unroll
    for (int k = 0; k < 8; ++k) __builtin_amdgcn_raw_buffer_store_b128(v[k] ^ 1u, rd, voff, k * 4096, 0);
    // this workgroup's part of the bytes past n_read
    const int64_t tail = n_write - n_read;
    const int64_t per = ((tail + gridDim.x - 1) / gridDim.x + 15) / 16 * 16;
    const int64_t t0 = n_read + (int64_t)blockIdx.x * per;
    if (tail > 0 && t0 < n_write) {
        const int64_t len = (n_write - t0) < per ? (n_write - t0) : per;
        const __amdgpu_buffer_rsrc_t rt = stream_rsrc(dst + t0, len);
        const u32x4_t c = {(unsigned)blockIdx.x, 1u, 2u, 3u};
        for (int64_t o = voff; o < len; o += 256 * 16) __builtin_amdgcn_raw_buffer_store_b128(c, rt, (int)o, 0, 0);
    }
}
}  // namespace

hipError_t launch_diag_stream(const void* src, int64_t n_read, void* dst, int64_t n_write, hipStream_t stream) {
    const int64_t blocks = (n_read + kStreamChunk - 1) / kStreamChunk;
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(stream_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const uint8_t*>(src), n_read, static_cast<uint8_t*>(dst), n_write);
    return hipGetLastError();
}

}  // namespace bs
