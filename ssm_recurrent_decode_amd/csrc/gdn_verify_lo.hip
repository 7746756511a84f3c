// Instantiations of the GDN verify kernel for draft windows T = 1..4
// (own translation unit so the kernel variants compile in parallel).
#include "gdn.hpp"

namespace rssm_host {

int launch_gdn_verify_lo(int T, int D, const GdnReplayParams& p, int B, void* stream) {
  switch (T) {
    case 1: return D == 64 ? launch_gdn_window<64, 1>(p, B, stream) : launch_gdn_window<128, 1>(p, B, stream);
    case 2: return D == 64 ? launch_gdn_window<64, 2>(p, B, stream) : launch_gdn_window<128, 2>(p, B, stream);
    case 3: return D == 64 ? launch_gdn_window<64, 3>(p, B, stream) : launch_gdn_window<128, 3>(p, B, stream);
    case 4: return D == 64 ? launch_gdn_window<64, 4>(p, B, stream) : launch_gdn_window<128, 4>(p, B, stream);
    default: return RSSM_ENOTSUP;
  }
}

}  // namespace rssm_host
