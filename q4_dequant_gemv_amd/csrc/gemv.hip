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

// One iteration's weight bytes for one lane: per matrix and per owned group,
// the super-block header and the group's 32 code bytes.
template <int G, int NMAT>
struct RowLoads {
    uint4 hdr[NMAT][G];
    uint4 qa[NMAT][G];
    uint4 qb[NMAT][G];
};

// LPR lanes per row (power of two, <= 64), G groups per lane.  SWIGLU reads a
// second matrix `wu` of the same shape and writes silu(W x) * (Wu x).  XREG
// keeps the lane's activation limbs in registers for the whole kernel (G == 1);
// otherwise they are re-read from LDS for every row.
//
// Each wave walks its rows with two register buffers: the loads of the next
// row are in flight while the current row is decoded, multiplied and reduced,
// and the first row's loads are issued before the activations are prepared.
template <int LPR, int G, bool SWIGLU, bool XREG, int BLOCK, int MIN_WAVES>
__global__ __launch_bounds__(BLOCK, MIN_WAVES) void gemv_kernel(const uint8_t *__restrict__ w,
                                                                const uint8_t *__restrict__ wu, const float *x,
                                                                float *__restrict__ y, int64_t n, int ngroups,
                                                                int64_t row_bytes) {
    static_assert(G == 1 || LPR == 64, "several groups per lane only with a full wave per row");
    static_assert(!XREG || G == 1, "activation limbs held in registers for one group per lane");
    constexpr int NMAT = SWIGLU ? 2 : 1;
    constexpr int kRowsPerWave = kWave / LPR;
    constexpr int kWavesPerBlock = BLOCK / kWave;
    extern __shared__ __align__(16) unsigned char smem[];
    XGroup *xg = reinterpret_cast<XGroup *>(smem);

    const int lane = threadIdx.x & (kWave - 1);
    const int sub = lane % LPR;
    const int slot = lane / LPR;
    // Byte offsets of this lane's loads inside one wave iteration (rows
    // it*kRowsPerWave .. +kRowsPerWave-1), fixed for the whole kernel.  The
    // iteration's base address is wave-uniform (scalar registers), so the loop
    // rewrites no per-lane address registers while earlier loads are in flight.
    // Lanes past the row's last group (K/64 not a power of two) load group 0
    // again and ignore it.
    uint32_t off_hdr[G], off_qa[G];
    PairSelect psel[G];
    bool gok[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int j = sub + LPR * g;
        gok[g] = j < ngroups;
        const int jj = gok[g] ? j : 0;
        psel[g] = pair_select(jj & 3);
        off_hdr[g] = static_cast<uint32_t>(slot * row_bytes + (jj >> 2) * kBlockBytes);
        off_qa[g] = off_hdr[g] + 16u + 32u * static_cast<uint32_t>(jj & 3);
    }
    const uint8_t *mats[2] = {w, wu};
    // Loop control is 32-bit and scalar (the host keeps the iteration count
    // below 2^31): gfx9 has no 64-bit scalar compare, and a vector compare in
    // the loop would borrow registers that earlier memory operations still own.
    const int iter_bytes = kRowsPerWave * static_cast<int>(row_bytes);
    const int niters = static_cast<int>((n + kRowsPerWave - 1) / kRowsPerWave);
    const int tail_bytes = static_cast<int>(n - static_cast<int64_t>(niters - 1) * kRowsPerWave) *
                           static_cast<int>(row_bytes);

    // Loads of one iteration: unconditional, from a descriptor based at the
    // iteration's first row; rows past n read as zeros and are not stored.
    auto issue = [&](auto &b, int it) {
        const int64_t base = static_cast<int64_t>(it) * iter_bytes;
        const int left = niters - it;
        const int nrec = left > 1 ? iter_bytes : (left == 1 ? tail_bytes : 0);
#pragma unroll
        for (int mt = 0; mt < NMAT; ++mt) {
            const __amdgpu_buffer_rsrc_t r = stream_rsrc(mats[mt] + base, nrec);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                b.hdr[mt][g] = buffer_load16(r, off_hdr[g]);
                b.qa[mt][g] = buffer_load16(r, off_qa[g]);
                b.qb[mt][g] = buffer_load16(r, off_qa[g] + 16u);
            }
        }
    };

    const int nwaves = static_cast<int>(gridDim.x) * kWavesPerBlock;
    const int it0 = __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x) * kWavesPerBlock +
                                                   static_cast<int>(threadIdx.x >> 6));

    // activations first, then the first row's weights: waiting for the
    // activations (in issue order) then leaves the weight loads in flight
    constexpr int kXChunks = (64 * G * 16 + BLOCK - 1) / BLOCK;
    const XLoaded<kXChunks> xl = load_x<BLOCK, kXChunks>(x, ngroups);
    // keep the activation loads ahead of the weight loads (an empty asm with a
    // memory clobber: no instruction, only an ordering point for the compiler;
    // x is deliberately not __restrict__ so its loads cannot move across it)
    asm volatile("" ::: "memory");
    RowLoads<G, NMAT> bufa;
    RowLoads<G, XREG ? NMAT : 1> bufb;
    issue(bufa, it0);

    prepare_x<BLOCK, kXChunks>(xl, ngroups, xg);
    __syncthreads();

    XRegs xr[XREG ? 1 : 1];
    if constexpr (XREG) load_xregs(xg[gok[0] ? sub : 0], xr[0]);

    auto process = [&](const auto &b, int it) {
        const int64_t row = static_cast<int64_t>(it) * kRowsPerWave + slot;
        const bool rok = row < n;
        float acc[NMAT];
#pragma unroll
        for (int mt = 0; mt < NMAT; ++mt) {
            acc[mt] = 0.0f;
#pragma unroll
            for (int g = 0; g < G; ++g) {
                if (rok && gok[g]) {
                    GroupCodes c;
                    decode_group(b.hdr[mt][g], b.qa[mt][g], b.qb[mt][g], psel[g], c);
                    if constexpr (XREG) {
                        acc[mt] += xr[0].scale * group_dot(c, xr[0]);
                    } else {
                        const XGroup &xs = xg[sub + LPR * g];
                        acc[mt] += xs.scale * group_dot(c, xs);
                    }
                }
            }
            acc[mt] = lane_group_sum<LPR>(acc[mt]);
        }
        if (sub == 0 && rok) {
            if constexpr (SWIGLU) {
                y[row] = silu(acc[0]) * acc[1];
            } else {
                y[row] = acc[0];
            }
        }
    };

    // The loads are never inside a branch: at a control-flow join the wait
    // counters would have to assume the fewest loads in flight and drain the
    // prefetch.  Iterations past the end load nothing (0-byte descriptor).
    if constexpr (XREG) {
        for (int it = it0; it < niters; it += 2 * nwaves) {
            issue(bufb, it + nwaves);
            process(bufa, it);
            if (it + nwaves >= niters) break;
            issue(bufa, it + 2 * nwaves);
            process(bufb, it + nwaves);
        }
    } else {
        // G groups per lane already put G*48 bytes per lane in flight per row
        for (int it = it0; it < niters; it += nwaves) {
            if (it != it0) issue(bufa, it);
            process(bufa, it);
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

template <int LPR, int G, bool SWIGLU, bool XREG, int BLOCK, int MIN_WAVES>
hipError_t launch_fast(const uint8_t *w, const uint8_t *wu, const float *x, float *y, int64_t n, int64_t k,
                       hipStream_t stream) {
    auto kern = gemv_kernel<LPR, G, SWIGLU, XREG, BLOCK, MIN_WAVES>;
    const int ngroups = static_cast<int>(k / 64);
    const size_t lds = static_cast<size_t>(ngroups) * sizeof(XGroup);
    static std::atomic<int> cache[kMaxDevices];
    const int per_cu = resident_blocks_per_cu(kern, BLOCK, lds, cache);
    constexpr int kRowsPerWave = kWave / LPR;
    const int64_t niters = (n + kRowsPerWave - 1) / kRowsPerWave;
    const int64_t need = (niters + BLOCK / kWave - 1) / (BLOCK / kWave);
    const int64_t cap = static_cast<int64_t>(device_cu_count()) * per_cu;
    const int grid = static_cast<int>(need < cap ? need : cap);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(BLOCK), lds, stream, w, wu, x, y, n, ngroups,
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

// Launch shapes: threads per block and minimum resident waves per SIMD (the
// register budget).  Streams of several MB run best as one 1024-thread block
// per CU (4 waves per SIMD; more resident waves measured slower); small
// matrices, which finish in a few microseconds, start faster with 256-thread
// blocks (less activation preparation per block, more blocks).
#ifndef Q4K_LARGE_BLOCK
#define Q4K_LARGE_BLOCK 1024
#endif
#ifndef Q4K_LARGE_MINW
#define Q4K_LARGE_MINW 4
#endif
#ifndef Q4K_SMALL_BLOCK
#define Q4K_SMALL_BLOCK 256
#endif
#ifndef Q4K_SMALL_MINW
#define Q4K_SMALL_MINW 3
#endif
#ifndef Q4K_SWIGLU_BLOCK
#define Q4K_SWIGLU_BLOCK 512
#endif
#ifndef Q4K_SWIGLU_MINW
#define Q4K_SWIGLU_MINW 2
#endif
#ifndef Q4K_BIGK_BLOCK
#define Q4K_BIGK_BLOCK 1024
#endif
#ifndef Q4K_BIGK_MINW
#define Q4K_BIGK_MINW 4
#endif
// matrices below this many bytes use the small launch shape
#ifndef Q4K_SMALL_BYTES
#define Q4K_SMALL_BYTES (8 << 20)
#endif

template <int LPR, bool SWIGLU>
hipError_t dispatch_regx(const uint8_t *w, const uint8_t *wu, const float *x, float *y, int64_t n, int64_t k,
                         hipStream_t stream) {
    if constexpr (SWIGLU) {
        return launch_fast<LPR, 1, true, true, Q4K_SWIGLU_BLOCK, Q4K_SWIGLU_MINW>(w, wu, x, y, n, k, stream);
    } else {
        const int64_t bytes = n * (k / kBlockWeights) * kBlockBytes;
        if (bytes < Q4K_SMALL_BYTES) {
            return launch_fast<LPR, 1, false, true, Q4K_SMALL_BLOCK, Q4K_SMALL_MINW>(w, wu, x, y, n, k, stream);
        }
        return launch_fast<LPR, 1, false, true, Q4K_LARGE_BLOCK, Q4K_LARGE_MINW>(w, wu, x, y, n, k, stream);
    }
}

template <bool SWIGLU>
hipError_t dispatch(const uint8_t *w, const uint8_t *wu, const float *x, float *y, int64_t n, int64_t k,
                    hipStream_t stream) {
    const int64_t ngroups = k / 64;
    if (ngroups <= 4) return dispatch_regx<4, SWIGLU>(w, wu, x, y, n, k, stream);
    if (ngroups <= 8) return dispatch_regx<8, SWIGLU>(w, wu, x, y, n, k, stream);
    if (ngroups <= 16) return dispatch_regx<16, SWIGLU>(w, wu, x, y, n, k, stream);
    if (ngroups <= 32) return dispatch_regx<32, SWIGLU>(w, wu, x, y, n, k, stream);
    if (ngroups <= 64) return dispatch_regx<64, SWIGLU>(w, wu, x, y, n, k, stream);
    // two matrices' row buffers need twice the registers
    constexpr int BB = Q4K_BIGK_BLOCK;
    constexpr int BMW = SWIGLU ? 2 : Q4K_BIGK_MINW;
    constexpr int BBS = SWIGLU ? (BB > 512 ? 512 : BB) : BB;
    if (ngroups <= 128) return launch_fast<64, 2, SWIGLU, false, BBS, BMW>(w, wu, x, y, n, k, stream);
    if (ngroups <= 192) return launch_fast<64, 3, SWIGLU, false, BBS, BMW>(w, wu, x, y, n, k, stream);
    // beyond K = 12288 the per-row register buffers no longer fit
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
