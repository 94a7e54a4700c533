// stream.hip -- read-only HBM streaming reference at the decode kernel's access
// pattern (gfx950). Not a step of the method: it measures what one launch can
// stream from HBM when it does nothing with the bytes, so the decode kernel's
// rate can be read against a measured ceiling as well as the 8 TB/s peak.
//
// Same geometry as the M = 1 decode: blocks of 4 wavefronts, each wavefront
// reading 6 tiles of 768 contiguous bytes (lane l the 12 bytes at 12 l of each
// tile, one dwordx3 buffer load per tile), i.e. 4608 bytes per wavefront and
// 18432 per block, all loads issued before the first wait, with the decode's
// non-temporal cache policy. The words are
// combined by XOR, so nothing the hardware could skip; each wavefront stores
// one word.
#include "owq_device.h"
#include "owq_launch.h"

namespace owq {

namespace {

typedef uint32_t u32x3v __attribute__((ext_vector_type(3)));

constexpr int kTiles = 6;
constexpr int kWaveBytes = kTiles * 768;

__global__ __launch_bounds__(256) void k_stream_read(const uint8_t* src, int64_t bytes, uint32_t* sink)
{
    const int lane = threadIdx.x & 63;
    const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t off = w * kWaveBytes;
    const int64_t left = bytes - off;
    const int rec = left <= 0 ? 0 : (left < kWaveBytes ? (int)left : kWaveBytes);
    // bytes past the end of the buffer (the last wavefront's tail) read as 0
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(src) + (rec > 0 ? off : 0), (short)0, rec, 0x00020000);
    u32x3v v[kTiles];
#pragma unroll
    for (int t = 0; t < kTiles; t++)
        v[t] = __builtin_amdgcn_raw_buffer_load_b96(r, t * 768 + lane * 12, 0, 2);  // nt, as the decode's codes
    uint32_t x = 0;
#pragma unroll
    for (int t = 0; t < kTiles; t++)
        x ^= v[t].x ^ v[t].y ^ v[t].z;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1)
        x ^= (uint32_t)__shfl_xor((int)x, d);
    if (lane == 0 && rec > 0)
        sink[w] = x;
}

}  // namespace

int64_t stream_read_sink_words(int64_t bytes) { return (bytes + kWaveBytes - 1) / kWaveBytes; }

hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t s)
{
    const int64_t waves = stream_read_sink_words(bytes);
    const int64_t blocks = (waves + 3) / 4;
    hipLaunchKernelGGL(k_stream_read, dim3((unsigned)blocks), dim3(256), 0, s, (const uint8_t*)src, bytes, sink);
    return hipGetLastError();
}

}  // namespace owq
