// spa_vt.hip -- V re-laid out for the weights x V MFMA: per head, V^T with keys along rows.
//
// The attention launch multiplies V^T (dv x keys) by the transposed weights on MFMA, whose
// A operand gives each lane 8 keys of one V column. With V row-major ([N, dv], as the
// caller passes it) those 8 values are 8 rows apart, and reading them from LDS needs the
// transposing LDS read, which moves about a quarter of the bytes per clock of a plain
// 16-byte read. This launch writes, once per call, Vt[bh][c][k] = V[bh][k'][c] with the keys
// of every 16-key group stored in the order 0-3, 8-11, 4-7, 12-15 (the order in which the
// score accumulator holds them: a lane of half h holds keys 4h..4h+3 and 8+4h..8+4h+3 of each
// 16), and rows zero-padded to a multiple of 64 keys. Every A operand of the attention
// launch is then one 16-byte read. Cost: one read and one write of V, at HBM speed.
#include "spa_device.h"
#include "spa_internal.h"

namespace spa {
namespace {

constexpr int kVtThreads = 256;

// Position p (0..15) of a 16-key group holds key vt_key(p).
__device__ __forceinline__ int vt_key(int p) {
    const int h = p >> 3, j = p & 7;
    return 8 * (j >> 2) + 4 * h + (j & 3);
}

// One workgroup per (head, 64-key tile): V rows in with 16-byte loads, through LDS, V^T rows
// out with 16-byte stores.
template <int DV>
__global__ __launch_bounds__(kVtThreads) void vt_kernel(const uint16_t* __restrict__ V,
                                                        uint16_t* __restrict__ Vt, int N,
                                                        int Np, int ntiles) {
    constexpr int PITCH = DV + 8;  // LDS row pitch (elements): 16 bytes of padding
    constexpr int CH = DV / 8;     // 16-byte chunks per V row
    __shared__ __attribute__((aligned(16))) uint16_t s[kVtTileKeys * PITCH];

    const int bh = blockIdx.x / ntiles;
    const int k0 = (blockIdx.x - bh * ntiles) * kVtTileKeys;
    const uint16_t* Vh = V + (size_t)bh * N * DV;
    for (int c = threadIdx.x; c < kVtTileKeys * CH; c += kVtThreads) {
        const int r = c / CH, ch = c - r * CH;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (k0 + r < N) v = *reinterpret_cast<const u32x4*>(Vh + (size_t)(k0 + r) * DV + ch * 8);
        *reinterpret_cast<u32x4*>(s + r * PITCH + ch * 8) = v;
    }
    __syncthreads();
    uint16_t* Vth = Vt + (size_t)bh * DV * Np + k0;
    for (int c = threadIdx.x; c < DV * (kVtTileKeys / 8); c += kVtThreads) {
        const int col = c >> 3, ch = c & 7;  // V column, 16-byte chunk of the 64-key row
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int p0 = 8 * (ch & 1) + 2 * i;  // position within the 16-key group
            const int kk = 16 * (ch >> 1);
            const uint32_t lo = s[(kk + vt_key(p0)) * PITCH + col];
            const uint32_t hi = s[(kk + vt_key(p0 + 1)) * PITCH + col];
            w[i] = lo | (hi << 16);
        }
        *reinterpret_cast<u32x4*>(Vth + (size_t)col * Np + ch * 8) = w;
    }
}

template <int DV>
hipError_t launch(const void* V, void* Vt, int BH, int N, hipStream_t stream) {
    const int Np = vt_padded_keys(N);
    const long long blocks = (long long)BH * (Np / kVtTileKeys);
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    vt_kernel<DV><<<dim3((unsigned)blocks), kVtThreads, 0, stream>>>(
        static_cast<const uint16_t*>(V), static_cast<uint16_t*>(Vt), N, Np, Np / kVtTileKeys);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_vt_bf16(const void* V, void* Vt, int BH, int N, int dv, hipStream_t stream) {
    switch (dv) {
        case 64: return launch<64>(V, Vt, BH, N, stream);
        case 128: return launch<128>(V, Vt, BH, N, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace spa
