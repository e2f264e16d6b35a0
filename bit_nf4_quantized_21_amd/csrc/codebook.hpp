#pragma once

namespace qlora {
double normal_quantile(double p);
void build_codebook(float out[16]);
}  // namespace qlora
