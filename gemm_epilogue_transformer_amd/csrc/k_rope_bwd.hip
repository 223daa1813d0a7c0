// Backward of the RoPE epilogue of the QKV product (kucoin page, section "CODA: El
// epilogo esconde un tesoro", last paragraph: the reparameterisation covers RoPE and
// holds for the backward pass).  The forward wrote y = RoPE(z), z = r * acc with acc the
// unscaled product h . W'^T.  Given the upstream gradient dy, for each row m:
//   dL/dz = RoPE^T(dy): per rotated head, for i < 32 with (C, S) the angle's cos / sin
//     dL/dz[64c + i]      = dy[64c + i] C + dy[64c + i + 32] S
//     dL/dz[64c + i + 32] = dy[64c + i + 32] C - dy[64c + i] S
//   and dL/dz = dy in the columns past rot_cols (V);
//   dz[m, j] = bf16( r[m] dL/dz[m, j] )                           (row-major [M, N])
//   P[m, t]  = (1/r[m]) * sum over the columns j of tile t of dy[m, j] y[m, j]
// The rotation is orthogonal and never mixes tiles (a tile of 128 columns holds whole
// heads), so sum_j dL/dz_j acc_j = (1/r) sum_j dy_j y_j per tile: P is the RMSNorm
// backward's per-tile partial of c = sum_j dL/dz_j acc_j, in the layout of the SwiGLU
// backward's partials, computed from the saved output y (the backward of its bf16
// rounding taken as the identity) without recomputing the product.  dz then feeds the
// input-gradient GEMM and the token-contracting weight gradient unchanged.
//
// Tile: 64 rows x 128 columns, 256 threads.  A thread takes 4 (row, 8-column chunk)
// pairs: rows (thread / 16) + 16 i at chunk thread % 16, so 16 consecutive lanes cover
// one row's 128 columns.  A chunk lies in one half of one head (8 | 32), so it needs the
// partner chunk 32 columns away, which lane chunk ^ 4 of the same row holds (an 8-lane
// mirror, then a reversal inside each quad, as two data-parallel moves instead of a second
// load of dy), and 8 consecutive frequencies of the table row.  Every
// operand goes through buffer descriptors spanning the tile's rows; columns past N, and
// table rows outside [0, table_rows) (the forward read zero angles there), read at an
// offset beyond every range, i.e. zeros, and stores there are dropped.
#include "device_common.hpp"
#include "epilogue.hpp"
#include "launch.hpp"

namespace coda {

namespace {
constexpr int kRbRows = 64, kRbCols = 128;
constexpr int kRbPairs = kRbRows * (kRbCols / 8) / 256;   // (row, chunk) pairs per thread
}  // namespace

__global__ void __launch_bounds__(256)
k_rope_bwd(const uint16_t* __restrict__ DY, const uint16_t* __restrict__ Y, const float* __restrict__ R,
           const int32_t* __restrict__ POS, const float* __restrict__ COS, const float* __restrict__ SIN,
           uint16_t* __restrict__ DZ, float* __restrict__ P, int M, int N, int rot_cols, int table_rows,
           int tiles_n, int T) {
    const int tr = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
    const int m0 = tr * kRbRows, j0 = tn * kRbCols;
    const int tid = threadIdx.x;
    const int rows = min(kRbRows, M - m0);
    const uint32_t row_bytes = static_cast<uint32_t>(N) * 2u;
    const size_t base = static_cast<size_t>(m0) * N;
    const __amdgpu_buffer_rsrc_t dy_rsrc = make_buffer_rsrc(DY + base, static_cast<uint32_t>(rows) * row_bytes);
    const __amdgpu_buffer_rsrc_t y_rsrc = make_buffer_rsrc(Y + base, static_cast<uint32_t>(rows) * row_bytes);
    const __amdgpu_buffer_rsrc_t dz_rsrc = make_buffer_rsrc(DZ + base, static_cast<uint32_t>(rows) * row_bytes);
    const __amdgpu_buffer_rsrc_t r_rsrc = make_buffer_rsrc(R + m0, static_cast<uint32_t>(rows) * 4u);
    const bool any_rot = rot_cols > 0;
    const __amdgpu_buffer_rsrc_t pos_rsrc =
        make_buffer_rsrc(any_rot ? POS + m0 : nullptr, any_rot ? static_cast<uint32_t>(rows) * 4u : 0u);
    const uint32_t tbytes = any_rot ? static_cast<uint32_t>(table_rows) * 128u : 0u;
    const __amdgpu_buffer_rsrc_t cos_rsrc = make_buffer_rsrc(COS, tbytes);
    const __amdgpu_buffer_rsrc_t sin_rsrc = make_buffer_rsrc(SIN, tbytes);

    const int ch = tid & 15;
    const int j = j0 + 8 * ch;
    const bool col_in = j < N;
    const bool rotated = j < rot_cols;                       // rot_cols % 64 == 0: whole chunks
    const int i0 = j & 63;
    const bool first = i0 < 32;                              // first half of its head
    const uint32_t freq_off = static_cast<uint32_t>(i0 & 31) * 4u;

    i32x4_t dv[kRbPairs], yv[kRbPairs];
    f32x4_t c0[kRbPairs], c1[kRbPairs], s0[kRbPairs], s1[kRbPairs];
    float rv[kRbPairs];
    uint32_t off[kRbPairs];
#pragma unroll
    for (int it = 0; it < kRbPairs; ++it) {
        const uint32_t row = static_cast<uint32_t>((tid >> 4) + 16 * it);
        off[it] = col_in ? row * row_bytes + static_cast<uint32_t>(j) * 2u : kOobOffset;
        dv[it] = __builtin_amdgcn_raw_buffer_load_b128(dy_rsrc, off[it], 0, 0);
        yv[it] = __builtin_amdgcn_raw_buffer_load_b128(y_rsrc, off[it], 0, 0);
        rv[it] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r_rsrc, row * 4u, 0, 0));
        const int p = __builtin_amdgcn_raw_buffer_load_b32(pos_rsrc, row * 4u, 0, 0);
        const uint32_t toff = (rotated && p >= 0 && p < table_rows)
                                  ? static_cast<uint32_t>(p) * 128u + freq_off : kOobOffset;
        c0[it] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(cos_rsrc, toff, 0, 0));
        c1[it] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(cos_rsrc, toff + 16u, 0, 0));
        s0[it] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(sin_rsrc, toff, 0, 0));
        s1[it] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(sin_rsrc, toff + 16u, 0, 0));
    }
#pragma unroll
    for (int it = 0; it < kRbPairs; ++it) {
        const int row = (tid >> 4) + 16 * it;
        const float r = rv[it];
        float c = 0.0f;
        uint32_t o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            // lane l reads lane l ^ 4 of its 16-lane row: the 8-lane mirror takes l to
            // l ^ 7, the quad reversal (quad_perm 3,2,1,0) then flips the low two bits
            const int mirrored = __builtin_amdgcn_update_dpp(dv[it][e], dv[it][e], 0x141, 0xF, 0xF, false);
            const uint32_t xp = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(mirrored, mirrored, 0x1B, 0xF, 0xF, false));
            const uint32_t xd = static_cast<uint32_t>(dv[it][e]);
            const uint32_t xy = static_cast<uint32_t>(yv[it][e]);
            float g[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int f = 2 * e + hh;                     // frequency offset within the chunk
                const float d = bf16_bits_to_f32(static_cast<uint16_t>(hh ? xd >> 16 : xd & 0xFFFFu));
                const float q = bf16_bits_to_f32(static_cast<uint16_t>(hh ? xp >> 16 : xp & 0xFFFFu));
                const float yy = bf16_bits_to_f32(static_cast<uint16_t>(hh ? xy >> 16 : xy & 0xFFFFu));
                const float C = f < 4 ? c0[it][f] : c1[it][f - 4];
                const float S = f < 4 ? s0[it][f] : s1[it][f - 4];
                // own column j + f against its partner 32 columns away
                const float dl = rotated ? (first ? d * C + q * S : d * C - q * S) : d;
                g[hh] = r * dl;
                c += d * yy;
            }
            o[e] = pack_bf16x2(g[0], g[1]);
        }
        __builtin_amdgcn_raw_buffer_store_b128(i32x4_t{int(o[0]), int(o[1]), int(o[2]), int(o[3])}, dz_rsrc,
                                               off[it], 0, 0);
        // the row's 16 chunks sit in 16 consecutive lanes
        c = group_allreduce<16>(c, AddOp());
        if (ch == 0 && row < rows) P[static_cast<size_t>(m0 + row) * T + tn] = c / r;
    }
}

hipError_t launch_rope_bwd(int M, int N, const void* dy, const void* y, const float* r, const int32_t* pos,
                           const float* cos, const float* sin, int table_rows, int rot_cols, void* dz,
                           float* partials, hipStream_t stream) {
    const int tiles_r = (M + kRbRows - 1) / kRbRows, tiles_n = (N + kRbCols - 1) / kRbCols;
    const int T = static_cast<int>(swiglu_bwd_partials_per_row(N));
    hipLaunchKernelGGL(k_rope_bwd, dim3(static_cast<unsigned>(tiles_r) * tiles_n), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(dy), static_cast<const uint16_t*>(y), r, pos, cos, sin,
                       static_cast<uint16_t*>(dz), partials, M, N, rot_cols, table_rows, tiles_n, T);
    return hipGetLastError();
}

}  // namespace coda
