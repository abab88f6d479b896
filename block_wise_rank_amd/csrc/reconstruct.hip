// Rebuild X_hat_b = A_b B_b for a list of blocks.  Only the listed blocks are
// rebuilt (evolve.pub review of arXiv 2609.29913, FAQ).
//
// bf16 factors (the storage the method runs on): one workgroup of 4 waves per
// listed block, bf16 MFMA (16 x 16 x 32, fp32 accumulation; bf16 x bf16
// products are exact in fp32).  C (token x dim) = A (token x rank) . B (rank x
// dim): both operands need 8 consecutive ranks per lane but are stored
// rank-major, so B (once) and each 32-token tile of A^T are staged in LDS and
// read with transposing LDS loads.  Wave w keeps the B fragments of dims
// 32 w .. 32 w + 31 in registers; the A^T tiles are double-buffered through
// registers; each output tile goes through LDS so that every row is written
// with 16-byte stores.
//
// fp32, INT8, 4-bit and 2-bit factors: fp32 arithmetic on the decoded
// values, grid (listed block, 64-token tile), B_b and the 64-token slice of
// A_b^T staged in LDS, each thread accumulating 32 tokens of one column.
#include "common.hpp"
#include "kernels.hpp"

namespace milo {
namespace {

template <int F>
__device__ __forceinline__ float load_code(const uint8_t *p, int64_t idx) {
    if constexpr (F == kF32) return reinterpret_cast<const float *>(p)[idx];
    else if constexpr (F == kBF16) return bf16_bits_to_f32(reinterpret_cast<const uint16_t *>(p)[idx]);
    else return static_cast<float>(reinterpret_cast<const int8_t *>(p)[idx]);
}

// Element idx of a 4-bit code row starting at p (two's-complement nibbles,
// element 2k in the low nibble of byte k).
__device__ __forceinline__ float i4_code(const uint8_t *p, int64_t idx) {
    const int byte = p[idx >> 1];
    const int n = (idx & 1) ? (byte >> 4) : (byte & 15);
    return static_cast<float>(n >= 8 ? n - 16 : n);
}

// Element idx of a 2-bit code row starting at p (element 4k + j in bits 2j of
// byte k): the level 2c - 3 in units of the run's scale.
__device__ __forceinline__ float i2_code(const uint8_t *p, int64_t idx) {
    const int c = (p[idx >> 2] >> (2 * (idx & 3))) & 3;
    return static_cast<float>(2 * c - 3);
}

template <int F, int OUT>
__global__ __launch_bounds__(256) void reconstruct_kernel(
    const uint8_t *__restrict__ arena, const int32_t *__restrict__ rank,
    const int64_t *__restrict__ a_off, const int64_t *__restrict__ b_off,
    const float *__restrict__ a_scale, const float *__restrict__ b_scale, int T,
    const int32_t *__restrict__ ids, void *__restrict__ out, const int64_t *__restrict__ out_off) {
    __shared__ __align__(16) float Bs[kD * kD];
    __shared__ float As[kD * 64];
    const int n = blockIdx.x;
    const int id = ids[n];
    const int t0 = blockIdx.y * 64;
    const int tid = threadIdx.x;
    const int r = rank[id];
    const uint8_t *Ab = arena + a_off[id];
    const uint8_t *Bb = arena + b_off[id];
    for (int e = tid; e < r * kD; e += 256) {
        float v;
        if constexpr (F == kI4) {
            // code row i at Bb + i * d / 2, scales (r x d / 32) after the r code rows
            const float *bs = reinterpret_cast<const float *>(Bb + static_cast<int64_t>(r) * (kD / 2));
            v = i4_code(Bb, e) * bs[e / kI4Group];
        } else if constexpr (F == kI2) {
            const float *bs = reinterpret_cast<const float *>(Bb + static_cast<int64_t>(r) * (kD / 4));
            v = i2_code(Bb, e) * bs[e / kI4Group];
        } else {
            v = load_code<F>(Bb, e);
            if constexpr (F == kI8) v *= b_scale[static_cast<int64_t>(id) * kD + e / kD];
        }
        Bs[e] = v;
    }
    for (int e = tid; e < r * 64; e += 256) {
        const int i = e >> 6, tt = e & 63;
        float v;
        if constexpr (F == kI4) {
            const float *as = reinterpret_cast<const float *>(Ab + static_cast<int64_t>(r) * (T / 2));
            const int64_t idx = static_cast<int64_t>(i) * T + t0 + tt;
            v = i4_code(Ab, idx) * as[idx / kI4Group];
        } else if constexpr (F == kI2) {
            const float *as = reinterpret_cast<const float *>(Ab + static_cast<int64_t>(r) * (T / 4));
            const int64_t idx = static_cast<int64_t>(i) * T + t0 + tt;
            v = i2_code(Ab, idx) * as[idx / kI4Group];
        } else {
            v = load_code<F>(Ab, static_cast<int64_t>(i) * T + t0 + tt);
            if constexpr (F == kI8) v *= a_scale[static_cast<int64_t>(id) * T + t0 + tt];
        }
        As[e] = v;
    }
    __syncthreads();
    const int j = tid & 127, half = tid >> 7;
    float acc[32];
#pragma unroll
    for (int u = 0; u < 32; ++u) acc[u] = 0.f;
    for (int i = 0; i < r; ++i) {
        const float b = Bs[i * kD + j];
        const float *a = As + i * 64 + half * 32;
#pragma unroll
        for (int u = 0; u < 32; ++u) acc[u] = fmaf(a[u], b, acc[u]);
    }
    // element offset of this block's first output row
    const int64_t obase = out_off ? out_off[n] : static_cast<int64_t>(n) * T * kD;
    const int64_t row = t0 + half * 32;
#pragma unroll
    for (int u = 0; u < 32; ++u) {
        if constexpr (OUT == kF32)
            static_cast<float *>(out)[obase + (row + u) * kD + j] = acc[u];
        else
            static_cast<uint16_t *>(out)[obase + (row + u) * kD + j] = f32_to_bf16_bits(acc[u]);
    }
}

constexpr int kRT = 32;                  // tokens per tile
constexpr int kAP = 96;                  // LDS pitch (bytes) of a staged A^T row of one tile (64 B)
constexpr int kBP = 288;                 // LDS pitch (bytes) of a staged B row (256 B)
// The transposing loads of a half-wave touch 8 rows (r0 .. r0 + 3 and r0 + 8 ..
// r0 + 11) x 32 bytes; pitches that are odd multiples of 32 bytes spread them
// over all 32 banks twice, the minimum for 256 bytes.
static_assert(kAP % 64 == 32 && kBP % 64 == 32, "bank-spreading pitches");

__host__ __device__ constexpr int recon_bf16_lds(int out_elem) {
    return (kD * kBP > 2 * kD * kAP + kRT * kD * out_elem) ? kD * kBP : 2 * kD * kAP + kRT * kD * out_elem;
}

template <int OUT>
__global__ __launch_bounds__(256) void reconstruct_bf16_kernel(
    const uint8_t *__restrict__ arena, const int32_t *__restrict__ rank,
    const int64_t *__restrict__ a_off, const int64_t *__restrict__ b_off, int T,
    const int32_t *__restrict__ ids, void *__restrict__ out, const int64_t *__restrict__ out_off) {
    constexpr int OE = OUT == kF32 ? 4 : 2;  // output element bytes
    extern __shared__ __align__(16) uint8_t lds[];
    uint8_t *bst = lds;                      // B rows (prologue only)
    uint8_t *ast = lds;                      // [2][128 rows][kAP]: A^T tiles (after the prologue)
    uint8_t *ost = lds + 2 * kD * kAP;       // [32 tokens][128 dims] output tile

    const int n = blockIdx.x;
    const int id = ids[n];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c4 = lane >> 4, j = lane & 15;
    const int r = rank[id];
    uint8_t *ob = static_cast<uint8_t *>(out) + (out_off ? out_off[n] : static_cast<int64_t>(n) * T * kD) * OE;
    if (r == 0) {
        for (int64_t q = tid; q < static_cast<int64_t>(T) * kD * OE / 16; q += 256)
            reinterpret_cast<uint4 *>(ob)[q] = make_uint4(0u, 0u, 0u, 0u);
        return;
    }
    const int KS = (r + 31) >> 5, rpad = KS * 32;  // 32-rank k-steps
    const uint8_t *Ab = arena + a_off[id];
    const uint8_t *Bb = arena + b_off[id];

    // B rows 0 .. rpad - 1 (rows >= r zero) -> LDS
    for (int q = tid; q < rpad * 16; q += 256) {
        const int row = q >> 4, cc = q & 15;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (row < r) v = *reinterpret_cast<const uint4 *>(Bb + row * 256 + cc * 16);
        *reinterpret_cast<uint4 *>(bst + row * kBP + cc * 16) = v;
    }
    // A^T tile loads: rank row (q >> 2), 16-byte piece (q & 3) for q = tid and
    // tid + 256; rows >= r repeat row r - 1 (finite; their B rows are zero)
    const int qa0 = tid, qa1 = tid + 256;
    const int64_t ra0 = static_cast<int64_t>(min(qa0 >> 2, r - 1)) * T * 2 + (qa0 & 3) * 16;
    const int64_t ra1 = static_cast<int64_t>(min(qa1 >> 2, r - 1)) * T * 2 + (qa1 & 3) * 16;
    // (all 128 rows are staged; rows >= rpad are never read)
    const int sa0 = (qa0 >> 2) * kAP + (qa0 & 3) * 16, sa1 = (qa1 >> 2) * kAP + (qa1 & 3) * 16;
    uint4 a0, a1;
    auto load_a = [&](int tile) {
        a0 = *reinterpret_cast<const uint4 *>(Ab + ra0 + tile * kRT * 2);
        a1 = *reinterpret_cast<const uint4 *>(Ab + ra1 + tile * kRT * 2);
    };
    auto store_a = [&](int buf) {
        *reinterpret_cast<uint4 *>(ast + buf * kD * kAP + sa0) = a0;
        *reinterpret_cast<uint4 *>(ast + buf * kD * kAP + sa1) = a1;
    };
    load_a(0);
    __syncthreads();
    // B fragments of this wave's two 16-dim column tiles: lane (c, j) holds ranks
    // 32 ks + 8 c .. + 7 of dim 16 nt + j
    u16x8_t bfr[2][4];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            if (ks < KS) {
                const int nt = 2 * wave + u;
                const uint8_t *p0 = bst + (32 * ks + 8 * c4 + (j >> 2)) * kBP + (16 * nt + 4 * (j & 3)) * 2;
                bfr[u][ks] = cat8(lds_read_tr16(p0), lds_read_tr16(p0 + 4 * kBP));
            }
    __syncthreads();  // the B rows are dead: the A tiles and the output tile reuse the space

    const int n_tiles = T / kRT;
    for (int it = 0; it < n_tiles; ++it) {
        store_a(it & 1);
        if (it + 1 < n_tiles) load_a(it + 1);
        __syncthreads();
        const uint8_t *at = ast + (it & 1) * kD * kAP;
        f32x4_t acc[2][2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            acc[mt][0] = zero4();
            acc[mt][1] = zero4();
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                if (ks < KS) {
                    const uint8_t *p0 = at + (32 * ks + 8 * c4 + (j >> 2)) * kAP + (16 * mt + 4 * (j & 3)) * 2;
                    const u16x8_t afr = cat8(lds_read_tr16(p0), lds_read_tr16(p0 + 4 * kAP));
                    acc[mt][0] = mfma16x16x32(afr, bfr[0][ks], acc[mt][0]);
                    acc[mt][1] = mfma16x16x32(afr, bfr[1][ks], acc[mt][1]);
                }
        }
        // lane (c, j) holds tokens 16 mt + 4 c + i of dim 16 (2 wave + u) + j
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tok = 16 * mt + 4 * c4 + i, dim = 16 * (2 * wave + u) + j;
                    if constexpr (OUT == kF32)
                        *reinterpret_cast<float *>(ost + (tok * kD + dim) * 4) = acc[mt][u][i];
                    else
                        *reinterpret_cast<uint16_t *>(ost + (tok * kD + dim) * 2) = f32_to_bf16_bits(acc[mt][u][i]);
                }
        __syncthreads();
        uint8_t *dst = ob + static_cast<int64_t>(it) * kRT * kD * OE;
#pragma unroll
        for (int i = 0; i < kRT * kD * OE / 16 / 256; ++i) {
            const int q = tid + 256 * i;
            reinterpret_cast<uint4 *>(dst)[q] = reinterpret_cast<const uint4 *>(ost)[q];
        }
    }
}

}  // namespace

hipError_t launch_reconstruct(const void *arena, int f_type, const int32_t *rank,
                              const int64_t *a_off, const int64_t *b_off, const float *a_scale,
                              const float *b_scale, int block_len, const int32_t *ids, int n_ids,
                              void *out, const int64_t *out_off, int out_type, hipStream_t st) {
    if (n_ids <= 0) return hipSuccess;
    if (f_type == kBF16) {
        const int lds = recon_bf16_lds(out_type == kF32 ? 4 : 2);
        const void *fn = out_type == kF32 ? reinterpret_cast<const void *>(reconstruct_bf16_kernel<kF32>)
                                          : reinterpret_cast<const void *>(reconstruct_bf16_kernel<kBF16>);
        hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return e;
        const uint8_t *ar = static_cast<const uint8_t *>(arena);
        if (out_type == kF32)
            hipLaunchKernelGGL(reconstruct_bf16_kernel<kF32>, dim3(static_cast<unsigned>(n_ids)), dim3(256), lds,
                               st, ar, rank, a_off, b_off, block_len, ids, out, out_off);
        else
            hipLaunchKernelGGL(reconstruct_bf16_kernel<kBF16>, dim3(static_cast<unsigned>(n_ids)), dim3(256), lds,
                               st, ar, rank, a_off, b_off, block_len, ids, out, out_off);
        return hipGetLastError();
    }
    const dim3 grid(static_cast<unsigned>(n_ids), static_cast<unsigned>(block_len / 64));
    const uint8_t *ar = static_cast<const uint8_t *>(arena);
#define MILO_RECON(F, O)                                                                         \
    hipLaunchKernelGGL((reconstruct_kernel<F, O>), grid, dim3(256), 0, st, ar, rank, a_off,      \
                       b_off, a_scale, b_scale, block_len, ids, out, out_off)
    if (f_type == kF32) {
        if (out_type == kF32) MILO_RECON(kF32, kF32); else MILO_RECON(kF32, kBF16);
    } else if (f_type == kI4) {
        if (out_type == kF32) MILO_RECON(kI4, kF32); else MILO_RECON(kI4, kBF16);
    } else if (f_type == kI2) {
        if (out_type == kF32) MILO_RECON(kI2, kF32); else MILO_RECON(kI2, kBF16);
    } else {
        if (out_type == kF32) MILO_RECON(kI8, kF32); else MILO_RECON(kI8, kBF16);
    }
#undef MILO_RECON
    return hipGetLastError();
}

}  // namespace milo
