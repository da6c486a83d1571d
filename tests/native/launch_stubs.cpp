// Stand-ins for the device launchers of the HSTU library in the host-only
// sanitizer build (abi_sanitize.cpp): reaching one means a call passed
// validation and would have touched a GPU, which the driver never intends.
#include <cstdio>
#include <cstdlib>

#include "internal.h"

namespace {
[[noreturn]] void reached(const char* name) {
  std::fprintf(stderr, "device launcher %s reached in the host-only build\n", name);
  std::abort();
}
}  // namespace

namespace hstu {
hipError_t attn_static_scratch(void**) { reached("attn_static_scratch"); }
hipError_t launch_attn_bf16(const AttnArgs&, hipStream_t) { reached("launch_attn_bf16"); }
hipError_t launch_attn_f32(const AttnArgs&, hipStream_t) { reached("launch_attn_f32"); }
hipError_t launch_gemm_f32_mma(const GemmF32Args&, int, int, hipStream_t) { reached("launch_gemm_f32_mma"); }
hipError_t launch_proj_bf16(const ProjArgs&, hipStream_t) { reached("launch_proj_bf16"); }
hipError_t launch_proj_f32(const ProjArgs&, hipStream_t) { reached("launch_proj_f32"); }
hipError_t launch_out_bf16(const OutArgs&, hipStream_t) { reached("launch_out_bf16"); }
hipError_t launch_out_f32(const OutArgs&, hipStream_t) { reached("launch_out_f32"); }
hipError_t launch_norm_gate_bf16(const NormGateArgs&, hipStream_t) { reached("launch_norm_gate_bf16"); }
hipError_t launch_norm_gate_f32(const NormGateArgs&, hipStream_t) { reached("launch_norm_gate_f32"); }
hipError_t launch_layernorm_bf16(const LayerNormArgs&, hipStream_t) { reached("launch_layernorm_bf16"); }
hipError_t launch_layernorm_f32(const LayerNormArgs&, hipStream_t) { reached("launch_layernorm_f32"); }
hipError_t launch_attn_train_fwd(const BwdAttnArgs&, hipStream_t) { reached("launch_attn_train_fwd"); }
hipError_t launch_attn_bwd_f32(const BwdAttnArgs&, hipStream_t) { reached("launch_attn_bwd_f32"); }
hipError_t launch_attn_bwd_bf16(const BwdAttnArgs&, hipStream_t) { reached("launch_attn_bwd_bf16"); }
hipError_t launch_attn_fwd_bf16_rows(const BwdAttnArgs&, hipStream_t) { reached("launch_attn_fwd_bf16_rows"); }
hipError_t launch_to_bf16(const float*, uint16_t*, int64_t, hipStream_t) { reached("launch_to_bf16"); }
hipError_t launch_to_bf16_t(const float*, int64_t, int64_t, int, uint16_t*, int64_t, hipStream_t, uint16_t*, int64_t,
                            bool, float*) {
  reached("launch_to_bf16_t");
}
hipError_t launch_bf16_t(const uint16_t*, int64_t, int64_t, int, uint16_t*, int64_t, hipStream_t) {
  reached("launch_bf16_t");
}
hipError_t launch_gemm_bf16_f32(const GemmBf16Args&, hipStream_t) { reached("launch_gemm_bf16_f32"); }
hipError_t launch_to_bf16x3(const float*, int64_t, int, uint16_t*, int, hipStream_t) {
  reached("launch_to_bf16x3");
}
hipError_t launch_sum_splits(const float*, int, int64_t, float*, hipStream_t) { reached("launch_sum_splits"); }
hipError_t launch_gemm_f32s(const float*, int64_t, int64_t, const float*, int64_t, int64_t, float*, int64_t,
                            const float*, const float*, int, int, int64_t, int, hipStream_t) {
  reached("launch_gemm_f32s");
}
hipError_t launch_fill_zero_list(const ZeroList&, hipStream_t) { reached("launch_fill_zero_list"); }
hipError_t launch_ln1_bwd(const float*, const float*, const float*, const float*, float*, float*, float*,
                          int64_t, int, float, hipStream_t) {
  reached("launch_ln1_bwd");
}
hipError_t launch_colsum(const float*, int64_t, int64_t, int, float*, hipStream_t) { reached("launch_colsum"); }
hipError_t launch_ln_gate_fwd(const float*, const float*, const float*, const float*, float*, float*, float*,
                              uint16_t*, int64_t, int, float, hipStream_t) {
  reached("launch_ln_gate_fwd");
}
hipError_t launch_ln_gate_bwd(const float*, const float*, const float*, const float*, const float*,
                              const float*, float*, int64_t, float*, uint16_t*, float*, float*, int64_t, int,
                              hipStream_t) {
  reached("launch_ln_gate_bwd");
}
hipError_t launch_silu_bwd(float*, const float*, int64_t, hipStream_t) { reached("launch_silu_bwd"); }
hipError_t launch_silu_bwd_bf16(const float*, const float*, int64_t, int, uint16_t*, uint16_t*, int64_t, float*,
                                hipStream_t) {
  reached("launch_silu_bwd_bf16");
}
hipError_t launch_gather_rows(int64_t, int, const int64_t*, int64_t, const void*, void*, hipStream_t) {
  reached("launch_gather_rows");
}
hipError_t launch_cache_concat(const CacheConcatArgs&, hipStream_t) { reached("launch_cache_concat"); }
hipError_t launch_linear_bias_tables(float, float, int, int, int, float*, float*, hipStream_t) {
  reached("launch_linear_bias_tables");
}
hipError_t launch_embed_bf16(const EmbedArgs&, hipStream_t) { reached("launch_embed_bf16"); }
hipError_t launch_embed_f32(const EmbedArgs&, hipStream_t) { reached("launch_embed_f32"); }
}  // namespace hstu
