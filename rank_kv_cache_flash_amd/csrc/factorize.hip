// factorize.hip -- offline per-head factorisation W_h ~ A_h B_h.
//
// Each head's E x H slice of a projection is factored on its own at rank r
// (Arabic page section 2a, German page section 2A, Japanese page section 2.1),
// and the factors may then be refined against an error weighted elementwise
// by importance weights F (Arabic page section 2b, German page section 2B,
// Japanese page section 2.2).
//
// Truncated SVD, through the head's Gram matrix G = W_h^T W_h in fp64:
//   gram_kernel     partial G over chunks of rows (fp64 sums of fp32 inputs);
//   jacobi_kernel   one workgroup per head adds the partials into LDS and runs
//                   one-sided Jacobi (Hestenes' method) on the columns of X = G,
//                   H/2 disjoint column pairs at a time in round-robin
//                   tournament order.  At convergence the columns of X = G J
//                   are mutually orthogonal; G being symmetric positive
//                   semidefinite, J then holds its eigenvectors and column j
//                   of X equals lambda_j v_j.  So the eigenvalues are the
//                   column norms and the eigenvectors the normalised columns,
//                   and J is never stored (LDS holds X only).  The r largest
//                   are re-orthonormalised (classical Gram-Schmidt, two
//                   passes); a direction whose eigenvalue is at rounding level
//                   is replaced by the unit vector furthest from the span
//                   already chosen, so a rank-deficient head still gets
//                   orthonormal rows of B.  Signs: the largest-magnitude
//                   entry of every row of B is positive.
//   project_kernel  A_h = W_h B_h^T from the fp32 rows of B (fp64 sums), so
//                   the returned pair is consistent to fp32 rounding.
//
// Weighted refinement, alternating least squares with one wave per unknown
// vector: with B fixed, row e of A_h solves (B diag(F_e) B^T) a = B diag(F_e)
// W_e^T (als_rows_kernel); with A fixed, column j of B_h solves
// (A^T diag(F_j) A) b = A^T diag(F_j) W_j (als_cols_kernel).  Both build the
// r x r normal matrix in fp64 across the wave (lane (ti, tj) of an 8 x 8 grid
// owns an (r/8) x (r/8) tile) and solve it by Gauss-Jordan elimination
// without pivoting (the matrix is symmetric positive definite).
#include <math.h>

#include "wsvd_common.hpp"
#include "wsvd_internal.hpp"

namespace wsvd {
namespace {

constexpr int kGramRows = 32;     // rows staged per pass of gram_kernel
constexpr int kMaxSweeps = 40;    // Jacobi sweeps before giving up
constexpr int kProjRows = 32;     // rows of A per project_kernel block
constexpr int kAlsRowsPerWave = 8;
constexpr int kAlsChunk = 64;     // rows of A staged per pass of als_cols_kernel

// ---------------------------------------------------------------------------
// Gram matrix.  Block (c, h) sums W_h[e, :]^T W_h[e, :] over its chunk of
// rows; thread (ti, tj) of a 16 x 16 grid owns a TS x TS tile of G.
template <int H>
__global__ __launch_bounds__(256) void gram_kernel(const float* __restrict__ W, int E, int nh,
                                                   int rows_per_chunk, double* __restrict__ Gpart) {
    constexpr int TS = H / 16;
    constexpr int Q = H / 4;  // float4 per row
    __shared__ double sW[kGramRows][H];
    const int tid = threadIdx.x, ti = tid >> 4, tj = tid & 15;
    const int c = blockIdx.x, h = blockIdx.y;
    const size_t ld = (size_t)nh * H;
    const int e_begin = c * rows_per_chunk;
    const int e_end = min(E, e_begin + rows_per_chunk);

    double acc[TS][TS];
#pragma unroll
    for (int a = 0; a < TS; ++a)
#pragma unroll
        for (int b = 0; b < TS; ++b) acc[a][b] = 0.0;

    for (int e0 = e_begin; e0 < e_end; e0 += kGramRows) {
        __syncthreads();
#pragma unroll
        for (int it = 0; it < kGramRows * Q / 256; ++it) {
            const int idx = tid + 256 * it;
            const int row = idx / Q, c4 = idx % Q;
            const int e = e0 + row;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (e < e_end) v = *reinterpret_cast<const float4*>(W + (size_t)e * ld + (size_t)h * H + 4 * c4);
            sW[row][4 * c4 + 0] = v.x;
            sW[row][4 * c4 + 1] = v.y;
            sW[row][4 * c4 + 2] = v.z;
            sW[row][4 * c4 + 3] = v.w;
        }
        __syncthreads();
        for (int rr = 0; rr < kGramRows; ++rr) {
            double ui[TS], uj[TS];
#pragma unroll
            for (int a = 0; a < TS; ++a) ui[a] = sW[rr][ti * TS + a];
#pragma unroll
            for (int b = 0; b < TS; ++b) uj[b] = sW[rr][tj * TS + b];
#pragma unroll
            for (int a = 0; a < TS; ++a)
#pragma unroll
                for (int b = 0; b < TS; ++b) acc[a][b] = fma(ui[a], uj[b], acc[a][b]);
        }
    }
    double* G = Gpart + ((size_t)c * nh + h) * H * H;
#pragma unroll
    for (int a = 0; a < TS; ++a)
#pragma unroll
        for (int b = 0; b < TS; ++b) G[(size_t)(ti * TS + a) * H + tj * TS + b] = acc[a][b];
}

// DPP move of a double (two 32-bit halves).
template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
    const unsigned long long b = (unsigned long long)__double_as_longlong(v);
    const unsigned lo = (unsigned)__builtin_amdgcn_mov_dpp((int)(unsigned)b, CTRL, 0xF, 0xF, true);
    const unsigned hi = (unsigned)__builtin_amdgcn_mov_dpp((int)(unsigned)(b >> 32), CTRL, 0xF, 0xF, true);
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

// Sum over a row of 16 lanes.  Each level pairs lanes symmetrically and adds
// the same two operands on both sides, so every lane ends with the bitwise
// same total.
__device__ inline double group16_sum(double v) {
    v += dpp_d<kDppQuadXor1>(v);
    v += dpp_d<kDppQuadXor2>(v);
    v += dpp_d<kDppHalfMirror>(v);
    v += dpp_d<kDppRowMirror>(v);
    return v;
}

// Whole-block sum, deterministic (waves add in a fixed order).  Contains
// barriers: every thread of the block must call it.
template <int NT>
__device__ inline double block_sum(double v, double* red) {
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
    const int wave = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    double s = 0.0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) s += red[w];
    return s;
}

// ---------------------------------------------------------------------------
// One-sided Jacobi on X = G of one head; writes B rows, singular values and
// the sweep count.  8H threads: lane group g (16 lanes) handles column pair g
// of each tournament round, lane l of the group rows l, l + 16, ... (so a
// group reads 128 contiguous bytes per access).  Columns are CS doubles apart
// (padded: consecutive columns start 8 banks apart).
template <int H>
__global__ __launch_bounds__(8 * H) void jacobi_kernel(const double* __restrict__ Gpart, int nchunks, int nh,
                                                       int r, float* __restrict__ B, float* __restrict__ sigma,
                                                       int* __restrict__ sweeps_out) {
    constexpr int NT = 8 * H;
    constexpr int RPL = H / 16;
    constexpr int NP = H / 2;
    constexpr int CS = H + 4;
    __shared__ double X[H * CS];  // column j at X[j * CS, j * CS + H)
    __shared__ double lam[H];
    __shared__ double dots[H];
    __shared__ double red[NT / 64];
    __shared__ int order[H];
    __shared__ int flags[kMaxSweeps];
    __shared__ int pick;

    const int tid = threadIdx.x, g = tid >> 4, l = tid & 15;
    const int h = blockIdx.x;

    double fro = 0.0;
    for (int idx = tid; idx < H * H; idx += NT) {
        double s = 0.0;
        for (int c = 0; c < nchunks; ++c) s += Gpart[((size_t)c * nh + h) * H * H + idx];
        X[(idx / H) * CS + idx % H] = s;  // G is symmetric: row i doubles as column i
        fro = fma(s, s, fro);
    }
    for (int j = tid; j < kMaxSweeps; j += NT) flags[j] = 0;
    fro = sqrt(block_sum<NT>(fro, red));  // barriers inside publish X and flags

    // Pairs whose cosine is below tol are orthogonal to working accuracy;
    // columns no longer than `tiny` are rounding noise of an exact zero.
    const double tol = sqrt((double)H) * 0x1p-52;
    const double tiny = H * 0x1p-52 * fro;
    int used = -kMaxSweeps;
    for (int sw = 0; sw < kMaxSweeps; ++sw) {
        for (int k = 0; k < H - 1; ++k) {
            int p, q;
            if (g == 0) {
                p = k;
                q = H - 1;
            } else {
                p = (k + g) % (H - 1);
                q = (k + (H - 1) - g) % (H - 1);
            }
            double* cp = X + p * CS + l;
            double* cq = X + q * CS + l;
            double xp[RPL], xq[RPL];
            double a = 0.0, b = 0.0, c = 0.0;
#pragma unroll
            for (int i = 0; i < RPL; ++i) {
                xp[i] = cp[16 * i];
                xq[i] = cq[16 * i];
                a = fma(xp[i], xp[i], a);
                b = fma(xq[i], xq[i], b);
                c = fma(xp[i], xq[i], c);
            }
            a = group16_sum(a);
            b = group16_sum(b);
            c = group16_sum(c);
            const double na = sqrt(a), nb = sqrt(b);
            if (na > tiny && nb > tiny && fabs(c) > tol * na * nb) {
                // Rotation that zeroes the off-diagonal of [[a, c], [c, b]]
                // (the smaller root of t^2 + 2 zeta t - 1 = 0).
                const double zeta = (b - a) / (2.0 * c);
                double t;
                if (fabs(zeta) < 1e100)
                    t = (zeta >= 0.0 ? 1.0 : -1.0) / (fabs(zeta) + sqrt(fma(zeta, zeta, 1.0)));
                else
                    t = 0.5 / zeta;
                const double cs = 1.0 / sqrt(fma(t, t, 1.0));
                const double sn = cs * t;
#pragma unroll
                for (int i = 0; i < RPL; ++i) {
                    cp[16 * i] = cs * xp[i] - sn * xq[i];
                    cq[16 * i] = sn * xp[i] + cs * xq[i];
                }
                if (l == 0) flags[sw] = 1;
            }
            __syncthreads();
        }
        if (flags[sw] == 0) {
            used = sw + 1;
            break;
        }
    }

    // Eigenvalues = column norms; order them (descending, ties by index).
    for (int j = g; j < H; j += NP) {
        double s = 0.0;
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            const double v = X[j * CS + l + 16 * i];
            s = fma(v, v, s);
        }
        s = group16_sum(s);
        if (l == 0) lam[j] = s == s ? sqrt(s) : -1.0;  // NaN input: ordered last
    }
    __syncthreads();
    if (tid < H) {
        const double mine = lam[tid];
        int rank = 0;
        for (int i = 0; i < H; ++i) {
            const double o = lam[i];
            rank += (o > mine || (o == mine && i < tid)) ? 1 : 0;
        }
        order[rank] = tid;
    }
    __syncthreads();
    const double thr = lam[order[0]] * H * 0x1p-52;
    if (tid < H) sigma[(size_t)h * H + tid] = (float)sqrt(lam[order[tid]]);
    if (sweeps_out != nullptr && tid == 0) sweeps_out[h] = used;

    // Orthonormal basis of the r leading directions, in order.
    for (int k = 0; k < r; ++k) {
        const int j = order[k];
        double* cj = X + j * CS;
        if (!(lam[j] > thr)) {
            // Completion: the unit vector with the largest component outside
            // span(v_0 .. v_{k-1}) (first index on ties).
            if (tid < H) {
                double s = 0.0;
                for (int kk = 0; kk < k; ++kk) {
                    const double v = X[order[kk] * CS + tid];
                    s = fma(v, v, s);
                }
                dots[tid] = 1.0 - s;
            }
            __syncthreads();
            if (tid == 0) {
                int m = 0;
                for (int i = 1; i < H; ++i)
                    if (dots[i] > dots[m]) m = i;
                pick = m;
            }
            __syncthreads();
            if (tid < H) cj[tid] = tid == pick ? 1.0 : 0.0;
        }
        __syncthreads();
        for (int pass = 0; pass < 2; ++pass) {
            for (int kk = g; kk < k; kk += NP) {
                const double* v = X + order[kk] * CS + l;
                double s = 0.0;
#pragma unroll
                for (int i = 0; i < RPL; ++i) s = fma(v[16 * i], cj[l + 16 * i], s);
                s = group16_sum(s);
                if (l == 0) dots[kk] = s;
            }
            __syncthreads();
            if (tid < H) {
                double x = cj[tid];
                for (int kk = 0; kk < k; ++kk) x = fma(-dots[kk], X[order[kk] * CS + tid], x);
                cj[tid] = x;
            }
            __syncthreads();
        }
        const double x = tid < H ? cj[tid] : 0.0;
        const double nrm = sqrt(block_sum<NT>(x * x, red));
        if (tid < H) cj[tid] = x / nrm;
        __syncthreads();
    }

    // Sign convention and output: row k of B_h is v_k with its
    // largest-magnitude entry (first on ties) made positive.
    for (int k = g; k < r; k += NP) {
        const double* v = X + order[k] * CS;
        double best = -1.0, val = 0.0;
        int at = H;
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            const double x = v[l + 16 * i];
            if (fabs(x) > best) {
                best = fabs(x);
                val = x;
                at = l + 16 * i;
            }
        }
#pragma unroll
        for (int m = 8; m >= 1; m >>= 1) {
            const double ob = __shfl_xor(best, m), ov = __shfl_xor(val, m);
            const int oa = __shfl_xor(at, m);
            if (ob > best || (ob == best && oa < at)) {
                best = ob;
                val = ov;
                at = oa;
            }
        }
        const double sgn = val < 0.0 ? -1.0 : 1.0;
        float* out = B + ((size_t)h * r + k) * H + l;
#pragma unroll
        for (int i = 0; i < RPL; ++i) out[16 * i] = (float)(sgn * v[l + 16 * i]);
    }
}

// ---------------------------------------------------------------------------
// A_h = W_h B_h^T.  Block (x, h): kProjRows rows; thread (row, kg) computes
// columns kg, kg + 8, ..., kg + 8 (NM - 1) of its row, NM = ceil(r / 8)
// (columns at or beyond r are zero in LDS and never stored).
template <int H, int NM>
__global__ __launch_bounds__(256) void project_kernel(const float* __restrict__ W, const float* __restrict__ B,
                                                      int E, int nh, int r, float* __restrict__ A) {
    constexpr int KP = 8 * NM;
    __shared__ float VT[H * KP];              // VT[i * KP + k] = B_h[k, i]
    __shared__ float sW[kProjRows][H + 1];    // +1: the 8 rows a wave reads sit in different banks
    const int tid = threadIdx.x, h = blockIdx.y;
    const int e0 = blockIdx.x * kProjRows;
    const size_t ld = (size_t)nh * H;
    for (int idx = tid; idx < KP * H; idx += 256) {
        const int k = idx / H, i = idx % H;
        VT[i * KP + k] = k < r ? B[((size_t)h * r + k) * H + i] : 0.f;
    }
    for (int idx = tid; idx < kProjRows * H; idx += 256) {
        const int row = idx / H, i = idx % H;
        const int e = e0 + row;
        sW[row][i] = e < E ? W[(size_t)e * ld + (size_t)h * H + i] : 0.f;
    }
    __syncthreads();
    const int row = tid >> 3, kg = tid & 7;
    double acc[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) acc[m] = 0.0;
#pragma unroll 4
    for (int i = 0; i < H; ++i) {
        const double w = sW[row][i];
#pragma unroll
        for (int m = 0; m < NM; ++m) acc[m] = fma(w, (double)VT[i * KP + kg + 8 * m], acc[m]);
    }
    const int e = e0 + row;
    if (e < E) {
        float* out = A + (size_t)e * nh * r + (size_t)h * r;
#pragma unroll
        for (int m = 0; m < NM; ++m)
            if (kg + 8 * m < r) out[kg + 8 * m] = (float)acc[m];
    }
}

template <int H, int NM>
static void launch_project_nm(const float* W, const float* B, int E, int nh, int r, float* A, hipStream_t st) {
    const dim3 grid((E + kProjRows - 1) / kProjRows, nh);
    hipLaunchKernelGGL((project_kernel<H, NM>), grid, dim3(256), 0, st, W, B, E, nh, r, A);
}

template <int H>
static void launch_project(const float* W, const float* B, int E, int nh, int r, float* A, hipStream_t st) {
    switch ((r + 7) / 8) {
        case 1: launch_project_nm<H, 1>(W, B, E, nh, r, A, st); break;
        case 2: launch_project_nm<H, 2>(W, B, E, nh, r, A, st); break;
        case 3: launch_project_nm<H, 3>(W, B, E, nh, r, A, st); break;
        case 4: launch_project_nm<H, 4>(W, B, E, nh, r, A, st); break;
        case 5: launch_project_nm<H, 5>(W, B, E, nh, r, A, st); break;
        case 6: launch_project_nm<H, 6>(W, B, E, nh, r, A, st); break;
        case 7: launch_project_nm<H, 7>(W, B, E, nh, r, A, st); break;
        case 8: launch_project_nm<H, 8>(W, B, E, nh, r, A, st); break;
        case 9: launch_project_nm<H, 9>(W, B, E, nh, r, A, st); break;
        case 10: launch_project_nm<H, 10>(W, B, E, nh, r, A, st); break;
        case 11: launch_project_nm<H, 11>(W, B, E, nh, r, A, st); break;
        case 12: launch_project_nm<H, 12>(W, B, E, nh, r, A, st); break;
        case 13: launch_project_nm<H, 13>(W, B, E, nh, r, A, st); break;
        case 14: launch_project_nm<H, 14>(W, B, E, nh, r, A, st); break;
        case 15: launch_project_nm<H, 15>(W, B, E, nh, r, A, st); break;
        default: launch_project_nm<H, 16>(W, B, E, nh, r, A, st); break;
    }
}

// ---------------------------------------------------------------------------
// Wave-level weighted least squares, r = 8 TS unknowns.  Lane (ti, tj) of the
// 8 x 8 lane grid owns M[ti TS + a][tj TS + b] and rhs[ti TS + a] (the rhs is
// kept identical across tj).
template <int TS>
struct WlsTile {
    double m[TS][TS];
    double rhs[TS];
};

// LDS hand-off between lanes of one wave: the fences keep the compiler from
// moving LDS accesses across and wait for the wave's own LDS traffic.
__device__ inline void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

template <int TS>
__device__ inline void wls_zero(WlsTile<TS>& T) {
#pragma unroll
    for (int a = 0; a < TS; ++a) {
        T.rhs[a] = 0.0;
#pragma unroll
        for (int b = 0; b < TS; ++b) T.m[a][b] = 0.0;
    }
}

// M += w u u^T, rhs += wy u.
template <int TS>
__device__ inline void wls_add(WlsTile<TS>& T, const double* u, double w, double wy, int ti, int tj) {
    double ui[TS], uj[TS];
#pragma unroll
    for (int a = 0; a < TS; ++a) ui[a] = u[ti * TS + a];
#pragma unroll
    for (int b = 0; b < TS; ++b) uj[b] = u[tj * TS + b];
#pragma unroll
    for (int a = 0; a < TS; ++a) {
        const double wu = w * ui[a];
#pragma unroll
        for (int b = 0; b < TS; ++b) T.m[a][b] = fma(wu, uj[b], T.m[a][b]);
        T.rhs[a] = fma(wy, ui[a], T.rhs[a]);
    }
}

// Gauss-Jordan elimination of [M | rhs]; afterwards M is diagonal and the
// solution is rhs_i / M_ii (read by the lanes with ti == tj).  buf holds
// 2 r + 1 doubles of this wave's LDS.
template <int TS>
__device__ inline void wls_solve(WlsTile<TS>& T, double* buf, int ti, int tj) {
    constexpr int R = 8 * TS;
    double* colb = buf;
    double* rowb = buf + R;
    double* rkb = buf + 2 * R;
    for (int kt = 0; kt < 8; ++kt) {
#pragma unroll
        for (int kb = 0; kb < TS; ++kb) {
            const int k = kt * TS + kb;
            if (tj == kt) {
#pragma unroll
                for (int a = 0; a < TS; ++a) colb[ti * TS + a] = T.m[a][kb];
            }
            if (ti == kt) {
#pragma unroll
                for (int b = 0; b < TS; ++b) rowb[tj * TS + b] = T.m[kb][b];
                if (tj == 0) rkb[0] = T.rhs[kb];
            }
            wave_lds_sync();
            const double ip = 1.0 / colb[k];
            double f[TS], rv[TS];
#pragma unroll
            for (int a = 0; a < TS; ++a) f[a] = (ti * TS + a == k) ? 0.0 : colb[ti * TS + a] * ip;
#pragma unroll
            for (int b = 0; b < TS; ++b) rv[b] = rowb[tj * TS + b];
            const double rk = rkb[0];
            wave_lds_sync();
#pragma unroll
            for (int a = 0; a < TS; ++a) {
#pragma unroll
                for (int b = 0; b < TS; ++b) T.m[a][b] = fma(-f[a], rv[b], T.m[a][b]);
                T.rhs[a] = fma(-f[a], rk, T.rhs[a]);
            }
        }
    }
}

// A step: row e of A_h from B_h.  Block (x, h), 4 waves, kAlsRowsPerWave
// consecutive rows per wave.
template <int H, int TS>
__global__ __launch_bounds__(256) void als_rows_kernel(const float* __restrict__ W, const float* __restrict__ F,
                                                       const float* __restrict__ B, int E, int nh,
                                                       float* __restrict__ A) {
    constexpr int R = 8 * TS;
    __shared__ double uT[H * R];         // uT[t * R + k] = B_h[k, t]
    __shared__ double wbuf[4][2 * H];    // per wave: F_e, F_e W_e
    __shared__ double piv[4][2 * R + 2];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int ti = lane >> 3, tj = lane & 7;
    const int h = blockIdx.y;
    const size_t ld = (size_t)nh * H;
    for (int idx = tid; idx < R * H; idx += 256) {
        const int k = idx / H, t = idx % H;
        uT[t * R + k] = B[((size_t)h * R + k) * H + t];
    }
    __syncthreads();
    double* wb = wbuf[wave];
    for (int it = 0; it < kAlsRowsPerWave; ++it) {
        const int e = (blockIdx.x * 4 + wave) * kAlsRowsPerWave + it;
        if (e >= E) break;
        for (int t = lane; t < H; t += 64) {
            const size_t off = (size_t)e * ld + (size_t)h * H + t;
            const double f = F[off];
            wb[t] = f;
            wb[H + t] = f * (double)W[off];
        }
        wave_lds_sync();
        WlsTile<TS> T;
        wls_zero(T);
        for (int t = 0; t < H; ++t) wls_add(T, uT + t * R, wb[t], wb[H + t], ti, tj);
        wls_solve(T, piv[wave], ti, tj);
        if (ti == tj) {
            float* out = A + (size_t)e * nh * R + (size_t)h * R + ti * TS;
#pragma unroll
            for (int a = 0; a < TS; ++a) out[a] = (float)(T.rhs[a] / T.m[a][a]);
        }
    }
}

// B step: column j of B_h from A_h.  Block (x, h), 4 waves, wave w solves
// column 4 x + w; rows of A_h stream through LDS kAlsChunk at a time.
template <int H, int TS>
__global__ __launch_bounds__(256) void als_cols_kernel(const float* __restrict__ W, const float* __restrict__ F,
                                                       const float* __restrict__ A, int E, int nh,
                                                       float* __restrict__ B) {
    constexpr int R = 8 * TS;
    __shared__ double sA[kAlsChunk][R];
    __shared__ double sw[kAlsChunk][4];
    __shared__ double swy[kAlsChunk][4];
    __shared__ double piv[4][2 * R + 2];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int ti = lane >> 3, tj = lane & 7;
    const int h = blockIdx.y, j0 = blockIdx.x * 4;
    const size_t ld = (size_t)nh * H;
    const size_t lda = (size_t)nh * R;
    WlsTile<TS> T;
    wls_zero(T);
    for (int e0 = 0; e0 < E; e0 += kAlsChunk) {
        __syncthreads();
        for (int idx = tid; idx < kAlsChunk * R; idx += 256) {
            const int row = idx / R, k = idx % R;
            const int e = e0 + row;
            sA[row][k] = e < E ? (double)A[(size_t)e * lda + (size_t)h * R + k] : 0.0;
        }
        {
            const int row = tid >> 2, cc = tid & 3;
            const int e = e0 + row;
            double f = 0.0, fy = 0.0;
            if (e < E) {
                const size_t off = (size_t)e * ld + (size_t)h * H + j0 + cc;
                f = F[off];
                fy = f * (double)W[off];
            }
            sw[row][cc] = f;
            swy[row][cc] = fy;
        }
        __syncthreads();
        for (int t = 0; t < kAlsChunk; ++t) wls_add(T, sA[t], sw[t][wave], swy[t][wave], ti, tj);
    }
    wls_solve(T, piv[wave], ti, tj);
    if (ti == tj) {
        const int j = j0 + wave;
#pragma unroll
        for (int a = 0; a < TS; ++a) B[((size_t)h * R + ti * TS + a) * H + j] = (float)(T.rhs[a] / T.m[a][a]);
    }
}

}  // namespace

int svd_num_chunks(int E, int nh) {
    // Enough (chunk, head) blocks to cover the CUs twice; at least 64 rows each.
    // (64-bit intermediates: E and nh may be any positive int here.)
    long c = (512L + nh - 1) / nh;
    const long cmax = ((long)E + 63) / 64;
    if (c > cmax) c = cmax;
    if (c < 1) c = 1;
    long rows = ((long)E + c - 1) / c;
    rows = (rows + kGramRows - 1) / kGramRows * kGramRows;
    return (int)(((long)E + rows - 1) / rows);
}

static int svd_rows_per_chunk(int E, int nh) {
    const long c = svd_num_chunks(E, nh);
    const long rows = ((long)E + c - 1) / c;
    return (int)((rows + kGramRows - 1) / kGramRows * kGramRows);
}

hipError_t launch_factorize_svd(const float* W, int E, int nh, int H, int r, float* A, float* B, float* sigma,
                                int* sweeps, double* Gpart, hipStream_t st) {
    const int nc = svd_num_chunks(E, nh);
    const int rpc = svd_rows_per_chunk(E, nh);
    const dim3 ggrid(nc, nh);
    if (H == 128) {
        hipLaunchKernelGGL((gram_kernel<128>), ggrid, dim3(256), 0, st, W, E, nh, rpc, Gpart);
        hipLaunchKernelGGL((jacobi_kernel<128>), dim3(nh), dim3(1024), 0, st, Gpart, nc, nh, r, B, sigma, sweeps);
        launch_project<128>(W, B, E, nh, r, A, st);
    } else if (H == 64) {
        hipLaunchKernelGGL((gram_kernel<64>), ggrid, dim3(256), 0, st, W, E, nh, rpc, Gpart);
        hipLaunchKernelGGL((jacobi_kernel<64>), dim3(nh), dim3(512), 0, st, Gpart, nc, nh, r, B, sigma, sweeps);
        launch_project<64>(W, B, E, nh, r, A, st);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int H, int TS>
static void launch_als_pair(bool rows, const float* W, const float* F, const float* in, int E, int nh, float* out,
                            hipStream_t st) {
    if (rows) {
        const int per_block = 4 * kAlsRowsPerWave;
        hipLaunchKernelGGL((als_rows_kernel<H, TS>), dim3((E + per_block - 1) / per_block, nh), dim3(256), 0, st, W,
                           F, in, E, nh, out);
    } else {
        hipLaunchKernelGGL((als_cols_kernel<H, TS>), dim3(H / 4, nh), dim3(256), 0, st, W, F, in, E, nh, out);
    }
}

template <int H>
static hipError_t launch_als_h(bool rows, const float* W, const float* F, const float* in, int E, int nh, int r,
                               float* out, hipStream_t st) {
    switch (r) {
        case 16: launch_als_pair<H, 2>(rows, W, F, in, E, nh, out, st); break;
        case 32: launch_als_pair<H, 4>(rows, W, F, in, E, nh, out, st); break;
        case 48: launch_als_pair<H, 6>(rows, W, F, in, E, nh, out, st); break;
        case 64: launch_als_pair<H, 8>(rows, W, F, in, E, nh, out, st); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_factorize_weighted(bool rows, const float* W, const float* F, const float* in, int E, int nh,
                                     int H, int r, float* out, hipStream_t st) {
    if (H == 128) return launch_als_h<128>(rows, W, F, in, E, nh, r, out, st);
    if (H == 64) return launch_als_h<64>(rows, W, F, in, E, nh, r, out, st);
    return hipErrorInvalidValue;
}

}  // namespace wsvd
