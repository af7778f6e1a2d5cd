// Batch-1 Q4_K GEMV and the fused gate/up SwiGLU GEMV.
//
// The operation is the fused dequant+GEMV over raw Q4K bytes of "Struct
// WgslForwardPass" (upload_q4k_weight) and the try_q4k_soa_gemv /
// try_q4k_soa_fused_swiglu entry points of the qualia_core_db cuda_lane
// module, at M == 1 (the decode phase of resolveMatmulPhase in
// "@simulatte/doppler 0.1.7 -> 0.1.8", matmul-selection.js).
//
// Design for gfx950.  At batch 1 every weight byte is used once, so the
// kernel is an HBM stream: each lane owns one 64-weight group (the code bytes
// of a sub-block pair, 32 contiguous bytes) of a row, plus the super-block's
// 16-byte header, and a row of K weights is covered by LPR = K/64 lanes (16,
// 32 or 64 at K = 1024, 2048, 4096; a lane owns G groups when K/64 > 64).
// Rows are handed to waves round-robin by a persistent grid sized to the
// resident capacity.
//
// Arithmetic per weight has to stay near one vector instruction, so the dot
// product is done in integers: each 64-activation group is converted once per
// workgroup to X = rint(x * 2^(21-e)) (e = exponent of the group's largest
// magnitude, |X| <= 2^22) and split into three signed bytes.  The codes are
// 0..15, so v_dot4_i32_i8 multiplies four codes by four activation bytes and
// accumulates exactly; per 8 weights that is 3 unpack + 6 dot instructions.
// Per sub-block s the exact integer S_s = sum q X combines the three limbs
// (|S_s| < 2^31 by construction), and the sub-block contributes
//     scale * (d*sc_s * S_s - dmin*m_s * sum_{e in s} X_e)
// in f32.  The min term uses the same integers X as the code term, so a
// sub-block whose weights are all zero still contributes zero.  Each x is
// represented to within 2^-22 of its group's largest magnitude, and the f32
// roundings are a few 2^-24 of the terms, so the error stays far inside the
// 2e-4 * sum|w x| bound unless, within one 64-activation group, the largest
// |x| exceeds the |w|-weighted typical |x| by several hundred times.
//
// Row partial sums are reduced across the LPR lanes of the row with
// cross-lane shuffles; the workgroup's activations are staged once in LDS and
// then held in registers for the whole row stream.
#include <float.h>
#include <math.h>

#include <atomic>

#include "launch.h"
#include "q4k_device.h"
#include "q4k_int_dot.h"

namespace q4k {

// LPR lanes per row (power of two, <= 64), G groups per lane; SWIGLU reads a
// second matrix `wu` of the same shape and writes silu(W x) * (Wu x).
template <int LPR, int G, bool SWIGLU, int BLOCK, int MIN_WAVES>
__global__ __launch_bounds__(BLOCK, MIN_WAVES) void gemv_kernel(const uint8_t *__restrict__ w,
                                                                const uint8_t *__restrict__ wu,
                                                                const float *__restrict__ x, float *__restrict__ y,
                                                                int64_t n, int ngroups, int64_t row_bytes) {
    static_assert(G == 1 || LPR == 64, "several groups per lane only with a full wave per row");
    constexpr int kRowsPerWave = kWave / LPR;
    constexpr int kWavesPerBlock = BLOCK / kWave;
    extern __shared__ __align__(16) unsigned char smem[];
    XGroup *xg = reinterpret_cast<XGroup *>(smem);

    prepare_x<BLOCK>(x, ngroups, xg);
    __syncthreads();

    const int lane = threadIdx.x & (kWave - 1);
    const int sub = lane % LPR;
    const int slot = lane / LPR;

    XRegs xr[G];
    int grp[G];
    int boff[G];
    bool gok[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int j = sub + LPR * g;
        gok[g] = j < ngroups;
        load_xregs(xg[gok[g] ? j : 0], xr[g]);
        grp[g] = j & 3;
        boff[g] = (j >> 2) * kBlockBytes;
    }

    const int64_t nwaves = static_cast<int64_t>(gridDim.x) * kWavesPerBlock;
    const int64_t niters = (n + kRowsPerWave - 1) / kRowsPerWave;
    for (int64_t it = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6); it < niters;
         it += nwaves) {
        const int64_t row = it * kRowsPerWave + slot;
        const bool rok = row < n;
        float acc = 0.0f, accu = 0.0f;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            if (rok && gok[g]) {
                const uint8_t *blk = w + row * row_bytes + boff[g];
                const uint4 hdr = load_stream16(blk);
                const uint4 qa = load_stream16(blk + 16 + 32 * grp[g]);
                const uint4 qb = load_stream16(blk + 32 + 32 * grp[g]);
                GroupCodes c;
                decode_group(hdr, qa, qb, grp[g], c);
                acc += xr[g].scale * group_dot(c, xr[g]);
                if constexpr (SWIGLU) {
                    const uint8_t *blku = wu + row * row_bytes + boff[g];
                    const uint4 hdru = load_stream16(blku);
                    const uint4 qau = load_stream16(blku + 16 + 32 * grp[g]);
                    const uint4 qbu = load_stream16(blku + 32 + 32 * grp[g]);
                    GroupCodes cu;
                    decode_group(hdru, qau, qbu, grp[g], cu);
                    accu += xr[g].scale * group_dot(cu, xr[g]);
                }
            }
        }
        acc = group_sum<LPR>(acc);
        if constexpr (SWIGLU) accu = group_sum<LPR>(accu);
        if (sub == 0 && rok) {
            if constexpr (SWIGLU) {
                y[row] = silu(acc) * accu;
            } else {
                y[row] = acc;
            }
        }
    }
}

// Any K: one wave per row, each lane dequantizes four weights at a time in f32
// and accumulates x * w with FMA; activations read straight from memory.
template <bool SWIGLU>
__global__ __launch_bounds__(256) void gemv_generic_kernel(const uint8_t *__restrict__ w,
                                                           const uint8_t *__restrict__ wu,
                                                           const float *__restrict__ x, float *__restrict__ y,
                                                           int64_t n, int64_t k, int64_t row_bytes) {
    const int lane = threadIdx.x & 63;
    const int64_t nwaves = static_cast<int64_t>(gridDim.x) * 4;
    const int64_t quads = k / 4;
    for (int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6); row < n; row += nwaves) {
        float acc[2] = {0.0f, 0.0f};
#pragma unroll
        for (int mat = 0; mat < (SWIGLU ? 2 : 1); ++mat) {
            const uint8_t *r = (mat == 0 ? w : wu) + row * row_bytes;
            for (int64_t t = lane; t < quads; t += 64) {
                const int64_t blk = t >> 6;
                const int e0 = static_cast<int>(t & 63) * 4;
                const uint8_t *b = r + blk * kBlockBytes;
                const uint4 hdr = *reinterpret_cast<const uint4 *>(b);
                const int g = e0 >> 6;
                const int rr = e0 & 63;
                const uint32_t codes = *reinterpret_cast<const uint32_t *>(b + 16 + 32 * g + (rr & 31));
                const uint32_t nib = (rr < 32) ? (codes & 0x0f0f0f0fu) : ((codes >> 4) & 0x0f0f0f0fu);
                int sc, m;
                scale_min(hdr.y, hdr.z, hdr.w, 2 * g + (rr >> 5), sc, m);
                const float dl = half_bits_to_float(hdr.x) * static_cast<float>(sc);
                const float ml = half_bits_to_float(hdr.x >> 16) * static_cast<float>(m);
                const float *xp = x + 4 * t;
#pragma unroll
                for (int b4 = 0; b4 < 4; ++b4) {
                    const float wv = dl * static_cast<float>((nib >> (8 * b4)) & 0xffu) - ml;
                    acc[mat] = fmaf(wv, xp[b4], acc[mat]);
                }
            }
            acc[mat] = group_sum<64>(acc[mat]);
        }
        if (lane == 0) y[row] = SWIGLU ? silu(acc[0]) * acc[1] : acc[0];
    }
}

namespace {

constexpr int kMaxDevices = 64;

template <typename Kernel>
int resident_blocks_per_cu(Kernel kern, int block, size_t lds, std::atomic<int> *cache) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kern, block, lds) != hipSuccess || nb < 1) nb = 1;
    cache[dev].store(nb, std::memory_order_relaxed);
    return nb;
}

template <int LPR, int G, bool SWIGLU>
hipError_t launch_fast(const uint8_t *w, const uint8_t *wu, const float *x, float *y, int64_t n, int64_t k,
                       hipStream_t stream) {
    constexpr int kBlock = (G == 1) ? 512 : 256;
    constexpr int kMinWaves = (G == 1) ? 4 : 2;
    auto kern = gemv_kernel<LPR, G, SWIGLU, kBlock, kMinWaves>;
    const int ngroups = static_cast<int>(k / 64);
    const size_t lds = static_cast<size_t>(ngroups) * sizeof(XGroup);
    static std::atomic<int> cache[kMaxDevices];
    const int per_cu = resident_blocks_per_cu(kern, kBlock, lds, cache);
    constexpr int kRowsPerWave = kWave / LPR;
    const int64_t niters = (n + kRowsPerWave - 1) / kRowsPerWave;
    const int64_t need = (niters + kBlock / kWave - 1) / (kBlock / kWave);
    const int64_t cap = static_cast<int64_t>(device_cu_count()) * per_cu;
    const int grid = static_cast<int>(need < cap ? need : cap);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kBlock), lds, stream, w, wu, x, y, n, ngroups,
                       (k / kBlockWeights) * kBlockBytes);
    return hipGetLastError();
}

template <bool SWIGLU>
hipError_t launch_generic(const uint8_t *w, const uint8_t *wu, const float *x, float *y, int64_t n, int64_t k,
                          hipStream_t stream) {
    const int64_t need = (n + 3) / 4;
    const int64_t cap = static_cast<int64_t>(device_cu_count()) * 8;
    const int grid = static_cast<int>(need < cap ? need : cap);
    hipLaunchKernelGGL(gemv_generic_kernel<SWIGLU>, dim3(grid), dim3(256), 0, stream, w, wu, x, y, n, k,
                       (k / kBlockWeights) * kBlockBytes);
    return hipGetLastError();
}

template <bool SWIGLU>
hipError_t dispatch(const uint8_t *w, const uint8_t *wu, const float *x, float *y, int64_t n, int64_t k,
                    hipStream_t stream) {
    const int64_t ngroups = k / 64;
    if (ngroups <= 4) return launch_fast<4, 1, SWIGLU>(w, wu, x, y, n, k, stream);
    if (ngroups <= 8) return launch_fast<8, 1, SWIGLU>(w, wu, x, y, n, k, stream);
    if (ngroups <= 16) return launch_fast<16, 1, SWIGLU>(w, wu, x, y, n, k, stream);
    if (ngroups <= 32) return launch_fast<32, 1, SWIGLU>(w, wu, x, y, n, k, stream);
    if (ngroups <= 64) return launch_fast<64, 1, SWIGLU>(w, wu, x, y, n, k, stream);
    if (ngroups <= 128) return launch_fast<64, 2, SWIGLU>(w, wu, x, y, n, k, stream);
    if (ngroups <= 192) return launch_fast<64, 3, SWIGLU>(w, wu, x, y, n, k, stream);
    // beyond K = 12288 the per-lane activations no longer fit in registers
    return launch_generic<SWIGLU>(w, wu, x, y, n, k, stream);
}

}  // namespace

hipError_t launch_gemv(const uint8_t *w, const uint8_t *w_up, const float *x, float *y, int64_t n, int64_t k,
                       hipStream_t stream) {
    if (n == 0) return hipSuccess;
    if (k == 0) return launch_fill_zero(y, n, stream);
    if (w_up != nullptr) return dispatch<true>(w, w_up, x, y, n, k, stream);
    return dispatch<false>(w, nullptr, x, y, n, k, stream);
}

}  // namespace q4k
