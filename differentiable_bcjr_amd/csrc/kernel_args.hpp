// kernel_args.hpp -- argument blocks passed by value from the C-ABI to the three kernels.
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace bcjr {

struct SoftArgs {
    const float* w;        // [B, n]
    const float* cb;       // [2^L]
    int64_t B;
    int n;
    float scale;           // sqrt(log2(e) / T)
    const int32_t* sigma;  // [B] or nullptr
    float* w_soft;         // [B, n]
    float* log_z;          // [B] or nullptr
    unsigned char* ws;
    size_t slot_bytes;
    int32_t sigma_enum;    // nonzero: sequence v decodes row v >> L with sigma = v mod 2^L (sigma ignored)
    int32_t ckpt;          // 0: every forward message row on the tape; c > 0: every c-th row (checkpoint kernels)
};

struct GradArgs {
    const float* w;        // [B, n]
    const float* cb;       // [2^L]
    const float* g;        // [B, n] upstream dL/dw_soft
    int64_t B;
    int n;
    float scale;           // sqrt(log2(e) / T)
    float two_over_T;
    const int32_t* sigma;  // [B] or nullptr
    float* grad;           // [B, n]
    float* w_soft;         // [B, n] or nullptr
    unsigned char* ws;
    size_t slot_bytes;
    int32_t sigma_enum;    // nonzero: sequence v decodes row v >> L with sigma = v mod 2^L (sigma ignored)
    int32_t ckpt;          // 0: every forward message row on the tape; c > 0: every c-th row (checkpoint kernels)
};

struct ViterbiArgs {
    const float* w;        // [rows, n]
    const float* cb;       // [2^L]
    int64_t B;             // sequences decoded (rows, or rows * 2^L with sigma_enum)
    int n;
    const int32_t* sigma;  // [B] or nullptr
    int32_t* states;       // [B, n], or nullptr for costs only (no traceback; w_hard must be nullptr too)
    float* w_hard;         // [B, n] or nullptr
    float* cost;           // [B] or nullptr
    unsigned char* ws;
    size_t slot_bytes;
    int32_t rot;           // sequence b emits w[b, (t + rot) mod n] at step t (0 <= rot < n)
    int32_t sigma_enum;    // nonzero: sequence v decodes row v >> L with sigma = v mod 2^L (sigma ignored)
};

// The general trellis (any k with 2k <= L, V weights per step): one argument block for its three kernels.
struct GenArgs {
    const float* w;        // [B, n V]
    const float* cb;       // [2^L, V]
    const float* g;        // [B, n V] upstream dL/dw_soft (gradient only)
    int64_t B;
    int n;                 // trellis steps
    int L;
    float scale;           // sqrt(log2(e) / T) (soft and gradient)
    float two_over_T;
    const int32_t* sigma;  // [B] or nullptr
    float* w_soft;         // [B, n V] (soft: required; gradient: optional)
    float* log_z;          // [B] or nullptr (soft)
    float* grad;           // [B, n V] (gradient)
    int32_t* states;       // [B, n] (Viterbi), or nullptr for costs only (no traceback; w_hard must be nullptr)
    float* w_hard;         // [B, n V] or nullptr (Viterbi)
    float* cost;           // [B] or nullptr (Viterbi)
    unsigned char* ws;
    size_t slot_bytes;
    int32_t dbl;           // LDS messages double-buffered (else one buffer, inputs read before outputs are written)
    int32_t ckpt;          // 0: every forward message row on the tape; c > 0: every c-th row, the backward pass
                           // recomputes each c-step segment from its checkpoint (soft codeword and gradient)
    int32_t sigma_enum;    // nonzero: sequence v decodes row v >> L with sigma = v mod 2^L (sigma ignored)
    int32_t nsq;           // Viterbi: sequences decoded together by one workgroup (1, or 2 where the plan pairs them)
    int32_t qg;            // gradients: nonzero puts the Q^ message in the workspace (its two messages exceed LDS)
};

}  // namespace bcjr
