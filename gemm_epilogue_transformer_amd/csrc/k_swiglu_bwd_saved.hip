// SwiGLU backward from a saved pre-activation (the forward kept z = r * (h . W'^T)), so no
// product is recomputed: for each row m and gate column j with g = z[m, j], u = z[m, F+j]
// and the upstream gradient d = dy[m, j],
//   dg = d u s (1 + g (1 - s)),   du = d g s,   s = sigma(g)
//   dz[m, j] = bf16( r[m] dg ),   dz[m, F+j] = bf16( r[m] du )       (row-major [M, 2F])
//   dzt[j, m] = dz[m, j]                                            (token-contiguous [2F, M])
//   P[m, t]  = (1/r[m]) * sum over the gate columns j of tile t of (dg g + du u)
// P has the layout the input-gradient path reduces (tiles of 128 gate columns), and
// (1/r) (dg g + du u) = dL/dz . acc with acc = z / r the unscaled product: the backward of
// the row scale in the same form as the recomputing kernel's epilogue (kucoin page,
// section "CODA: El epilogo esconde un tesoro": the backward inherits the forward's
// blockwise structure).  The transposed copy is what the token-contracting weight
// gradient reads; writing it here replaces a separate transpose pass.
//
// Tile: 64 rows x 128 gate columns (+ the 128 up columns), 256 threads.  A thread takes 4
// (row, 8-column chunk) pairs: rows (thread / 16) + 16 i of the tile at chunk thread % 16,
// so 16 consecutive lanes cover one row's 128 gate columns.  All operands go through
// buffer descriptors spanning the tile's rows, with columns past F sent to an offset
// beyond every range: reads outside the matrix return zeros and stores there are
// dropped, so the kernel has no branches around its memory operations and issues the
// loads of all 4 pairs (12 x 16 bytes of z and dy per thread) before the first wait.
// With the transpose, the bf16 dz tile is also staged in LDS (16-byte chunks
// XOR-swizzled by row / 8) and written transposed: 8 consecutive lanes write the 8
// 16-byte runs of one dzt row; without it the kernel takes no LDS.
#include "device_common.hpp"
#include "epilogue.hpp"
#include "launch.hpp"

namespace coda {

namespace {
constexpr int kSbRows = 64, kSbGate = 128, kSbCols = 2 * kSbGate;   // tile: rows x (gate + up) columns
constexpr int kSbPairs = kSbRows * (kSbGate / 8) / 256;             // (row, chunk) pairs per thread
}  // namespace

template <bool TR>
__global__ void __launch_bounds__(256)
k_swiglu_bwd_saved(const uint16_t* __restrict__ Z, const uint16_t* __restrict__ DY, const float* __restrict__ R,
                   uint16_t* __restrict__ DZ, uint16_t* __restrict__ DZT, float* __restrict__ P, int M, int F,
                   int tiles_f, int T) {
    __shared__ __attribute__((aligned(16))) uint16_t st[TR ? kSbRows : 1][kSbCols];
    const int tr = blockIdx.x / tiles_f, tf = blockIdx.x % tiles_f;
    const int m0 = tr * kSbRows, j0 = tf * kSbGate;
    const int tid = threadIdx.x;
    const int rows = min(kSbRows, M - m0);
    const uint32_t zrow = static_cast<uint32_t>(F) * 4u, drow = static_cast<uint32_t>(F) * 2u;
    const size_t zbase = static_cast<size_t>(m0) * 2 * F, dbase = static_cast<size_t>(m0) * F;
    const __amdgpu_buffer_rsrc_t z_rsrc = make_buffer_rsrc(Z + zbase, static_cast<uint32_t>(rows) * zrow);
    const __amdgpu_buffer_rsrc_t dz_rsrc = make_buffer_rsrc(DZ + zbase, static_cast<uint32_t>(rows) * zrow);
    const __amdgpu_buffer_rsrc_t dy_rsrc = make_buffer_rsrc(DY + dbase, static_cast<uint32_t>(rows) * drow);
    const __amdgpu_buffer_rsrc_t r_rsrc = make_buffer_rsrc(R + m0, static_cast<uint32_t>(rows) * 4u);
    const int ch = tid & 15;
    const int j = j0 + 8 * ch;
    const bool col_in = j < F;
    i32x4_t zg[kSbPairs], zu[kSbPairs], dv[kSbPairs];
    float rv[kSbPairs];
    uint32_t goff[kSbPairs], uoff[kSbPairs];
#pragma unroll
    for (int it = 0; it < kSbPairs; ++it) {
        const uint32_t row = static_cast<uint32_t>((tid >> 4) + 16 * it);
        goff[it] = col_in ? row * zrow + static_cast<uint32_t>(j) * 2u : kOobOffset;
        uoff[it] = col_in ? row * zrow + static_cast<uint32_t>(F + j) * 2u : kOobOffset;
        const uint32_t doff = col_in ? row * drow + static_cast<uint32_t>(j) * 2u : kOobOffset;
        zg[it] = __builtin_amdgcn_raw_buffer_load_b128(z_rsrc, goff[it], 0, 0);
        zu[it] = __builtin_amdgcn_raw_buffer_load_b128(z_rsrc, uoff[it], 0, 0);
        dv[it] = __builtin_amdgcn_raw_buffer_load_b128(dy_rsrc, doff, 0, 0);
        rv[it] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r_rsrc, row * 4u, 0, 0));
    }
#pragma unroll
    for (int it = 0; it < kSbPairs; ++it) {
        const int row = (tid >> 4) + 16 * it;
        const float r = rv[it];
        float c = 0.0f;
        uint32_t og[4], ou[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t xg = static_cast<uint32_t>(zg[it][e]), xu = static_cast<uint32_t>(zu[it][e]);
            const uint32_t xd = static_cast<uint32_t>(dv[it][e]);
            float dgo[2], duo[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const float g = bf16_bits_to_f32(static_cast<uint16_t>(hh ? xg >> 16 : xg & 0xFFFFu));
                const float u = bf16_bits_to_f32(static_cast<uint16_t>(hh ? xu >> 16 : xu & 0xFFFFu));
                const float d = bf16_bits_to_f32(static_cast<uint16_t>(hh ? xd >> 16 : xd & 0xFFFFu));
                const float s = __builtin_amdgcn_rcpf(1.0f + __expf(-g));
                const float dg = d * u * s * (1.0f + g * (1.0f - s));
                const float du = d * g * s;
                c += dg * g + du * u;
                dgo[hh] = r * dg;
                duo[hh] = r * du;
            }
            og[e] = pack_bf16x2(dgo[0], dgo[1]);
            ou[e] = pack_bf16x2(duo[0], duo[1]);
        }
        const i32x4_t vg = {int(og[0]), int(og[1]), int(og[2]), int(og[3])};
        const i32x4_t vu = {int(ou[0]), int(ou[1]), int(ou[2]), int(ou[3])};
        __builtin_amdgcn_raw_buffer_store_b128(vg, dz_rsrc, goff[it], 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(vu, dz_rsrc, uoff[it], 0, 0);
        if constexpr (TR) {
            // staged row `row`: gate chunk ch at logical chunk ch, up chunk at 16 + ch
            const int sw = (row >> 3) & 7;
            *reinterpret_cast<i32x4_t*>(&st[row][8 * (ch ^ sw)]) = vg;
            *reinterpret_cast<i32x4_t*>(&st[row][8 * ((16 + ch) ^ sw)]) = vu;
        }
        // the row's 16 chunks sit in 16 consecutive lanes
        c = group_allreduce<16>(c, AddOp());
        if (ch == 0 && row < rows) P[static_cast<size_t>(m0 + row) * T + tf] = c / r;
    }
    if constexpr (TR) {
        __syncthreads();
        // 256 staged columns x 8 chunks of 8 rows: lane group of 8 = one dzt row
#pragma unroll
        for (int it = 0; it < kSbCols * (kSbRows / 8) / 256; ++it) {
            const int idx = tid + 256 * it;
            const int col = idx >> 3, rc = idx & 7;            // staged column, 8-row chunk
            const int lc = col >> 3, within = col & 7;         // logical 16-byte chunk of the column
            const bool up = col >= kSbGate;
            const int jc = j0 + (up ? col - kSbGate : col);
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r0 = 8 * rc + 2 * e, r1 = r0 + 1;
                const uint16_t a = st[r0][8 * (lc ^ ((r0 >> 3) & 7)) + within];
                const uint16_t b = st[r1][8 * (lc ^ ((r1 >> 3) & 7)) + within];
                w[e] = static_cast<uint32_t>(a) | (static_cast<uint32_t>(b) << 16);
            }
            const int m = m0 + 8 * rc;
            if (jc < F && m < M)
                *reinterpret_cast<i32x4_t*>(DZT + static_cast<size_t>(up ? F + jc : jc) * M + m) =
                    i32x4_t{int(w[0]), int(w[1]), int(w[2]), int(w[3])};
        }
    }
}

hipError_t launch_swiglu_bwd_saved(int M, int F, const void* z, const void* dy, const float* r, void* dz,
                                   void* dzt, float* partials, hipStream_t stream) {
    const int tiles_r = (M + kSbRows - 1) / kSbRows, tiles_f = (F + kSbGate - 1) / kSbGate;
    const int T = static_cast<int>(swiglu_bwd_partials_per_row(F));
    const dim3 grid(static_cast<unsigned>(tiles_r) * tiles_f);
    auto* zp = static_cast<const uint16_t*>(z);
    auto* dyp = static_cast<const uint16_t*>(dy);
    auto* dzp = static_cast<uint16_t*>(dz);
    if (dzt)
        hipLaunchKernelGGL(k_swiglu_bwd_saved<true>, grid, dim3(256), 0, stream, zp, dyp, r, dzp,
                           static_cast<uint16_t*>(dzt), partials, M, F, tiles_f, T);
    else
        hipLaunchKernelGGL(k_swiglu_bwd_saved<false>, grid, dim3(256), 0, stream, zp, dyp, r, dzp, nullptr,
                           partials, M, F, tiles_f, T);
    return hipGetLastError();
}

}  // namespace coda
