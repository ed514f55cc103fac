// Device twin of the synth package's counter-based SplitMix64 generator.
//
// SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
// generators", OOPSLA 2014; constants of Vigna's public-domain splitmix64.c):
// output n of a stream with state s is mix(s + (n + 1) * 0x9E3779B97F4A7C15).
// The stream of MXFP4 tensor (layer, expert, matrix, part) has state
//   mix(seed + (id + 1) * 0x9E3779B97F4A7C15),
//   id = ((layer * 1025 + expert) * 3 + matrix) * 2 + part,
// code byte b is byte b % 8 (little-endian) of output b / 8, and scale byte i
// is lo + output i mod (hi - lo + 1).  Input generation only: no arithmetic of
// the MoE method lives here.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ull;

__host__ __device__ inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

__global__ void fill_kernel(uint8_t* dst, int n_experts, uint64_t bytes_per_expert, uint64_t seed,
                            int layer, int expert0, int matrix, int part, int lo, int hi) {
    const uint64_t per = part == 0 ? bytes_per_expert / 8 : bytes_per_expert;
    const uint64_t total = per * (uint64_t)n_experts;
    const uint64_t span = (uint64_t)(hi - lo + 1);
    for (uint64_t i = blockIdx.x * (uint64_t)blockDim.x + threadIdx.x; i < total;
         i += (uint64_t)gridDim.x * blockDim.x) {
        const uint64_t e = i / per, n = i % per;
        const uint64_t id = ((uint64_t)(layer * 1025 + expert0 + (int)e) * 3 + matrix) * 2 + part;
        const uint64_t state = mix64(seed + (id + 1) * kGolden);
        const uint64_t out = mix64(state + (n + 1) * kGolden);
        if (part == 0)
            reinterpret_cast<uint64_t*>(dst + e * bytes_per_expert)[n] = out;
        else
            dst[e * bytes_per_expert + n] = (uint8_t)(lo + out % span);
    }
}

}  // namespace

extern "C" {

// Fill n_experts consecutive tensors (experts expert0 .. expert0+n_experts-1)
// of `bytes_per_expert` bytes each.  part 0 = code bytes (bytes_per_expert a
// multiple of 8, dst 8-byte aligned), part 1 = scale bytes in [lo, hi].
// Returns 0, or -3 for bad sizes, -6 if the launch failed.
int synth_fill_mxfp4(uint8_t* dst, int n_experts, unsigned long long bytes_per_expert,
                     unsigned long long seed, int layer, int expert0, int matrix, int part, int lo,
                     int hi, void* stream) {
    if (!dst || n_experts < 1 || bytes_per_expert == 0 || matrix < 0 || matrix > 2 || part < 0 ||
        part > 1 || lo < 0 || hi > 255 || lo > hi || expert0 < 0 || expert0 + n_experts > 1025)
        return -3;
    if (part == 0 && (bytes_per_expert % 8 || reinterpret_cast<uintptr_t>(dst) % 8)) return -3;
    const uint64_t items = (part == 0 ? bytes_per_expert / 8 : bytes_per_expert) * n_experts;
    uint64_t blocks = (items + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), dst, n_experts,
                       (uint64_t)bytes_per_expert, (uint64_t)seed, layer, expert0, matrix, part, lo,
                       hi);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // extern "C"
