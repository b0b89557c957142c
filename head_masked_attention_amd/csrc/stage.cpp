// Host stage policy of libbsattn: whether the sparse stage serves an
// attention call, and at which budget.  Pure host code.
//
// SD.Next commit view, modules/attention/sparse:
//  - the stage-gating paragraph: the stage gates on the component role (self
//    attention), a minimum sequence length defaulting to the measured 8192
//    token crossover, and the absence of a token mask or causal flag, which a
//    block-only consumer cannot combine; budgets follow a precomputed per-step
//    schedule with at most two distinct values; enabling the feature with no
//    capable backend warns and leaves attention dense;
//  - the minimum-length paragraph: the default lives in the setting (8192),
//    0 means no floor, negative values stay unclaimed;
//  - the exclusion paragraph: a comma-separated denylist matched
//    case-insensitively against the architecture, the pipeline class and the
//    denoiser class, resolved once per model;
//  - the masked_block paragraph: calls carrying a token mask are served when
//    the backend composes a token mask with the block mask;
//  - the decline-log and no-layout paragraphs: the reason a call is declined,
//    and a sequence sparsified without a layout, are reported once per length.
#include <bsattn.h>

#include <cctype>
#include <cmath>
#include <mutex>
#include <set>
#include <map>
#include <string>
#include <tuple>
#include <vector>

struct bsattn_stage {
    bsattn_stage_config cfg;
    std::vector<std::string> exclude;      // lower-cased, trimmed, non-empty
    std::mutex lock;
    std::set<std::tuple<int32_t, int32_t, int64_t>> reported;   // (outcome, note, length)
    std::map<std::tuple<std::string, std::string, std::string>, bool> excluded;
};

namespace {

std::string lower_trim(const std::string& s) {
    size_t a = 0, b = s.size();
    while (a < b && std::isspace((unsigned char)s[a])) ++a;
    while (b > a && std::isspace((unsigned char)s[b - 1])) --b;
    std::string r = s.substr(a, b - a);
    for (char& c : r) c = (char)std::tolower((unsigned char)c);
    return r;
}

std::vector<std::string> split_list(const char* list) {
    std::vector<std::string> out;
    if (list == nullptr) return out;
    std::string cur;
    for (const char* p = list;; ++p) {
        if (*p == ',' || *p == '\0') {
            std::string t = lower_trim(cur);
            if (!t.empty()) out.push_back(t);
            cur.clear();
            if (*p == '\0') break;
        } else {
            cur.push_back(*p);
        }
    }
    return out;
}

bool budget_valid(double b) { return std::isfinite(b) && b > 0.0; }

}  // namespace

extern "C" {

const char* bsattn_stage_outcome_string(int32_t outcome) {
    switch (outcome) {
        case BSATTN_STAGE_SPARSE: return "served block-sparse";
        case BSATTN_DECLINE_DISABLED: return "sparse attention is disabled";
        case BSATTN_DECLINE_NO_BACKEND: return "no backend in the chain consumes a block mask; attention stays dense";
        case BSATTN_DECLINE_EXCLUDED: return "model is on the sparse-attention exclusion list";
        case BSATTN_DECLINE_NOT_SELF: return "not self attention";
        case BSATTN_DECLINE_SHORT: return "sequence shorter than the minimum length";
        case BSATTN_DECLINE_CAUSAL: return "causal attention cannot be served with a block mask";
        case BSATTN_DECLINE_TOKEN_MASK: return "token mask and no backend that composes it with a block mask";
    }
    return "unknown outcome";
}

bsattn_status bsattn_stage_create(const bsattn_stage_config* cfg, bsattn_stage** out) {
    if (cfg == nullptr || out == nullptr) return BSATTN_ERR_NULL;
    if (cfg->min_length < 0) return BSATTN_ERR_BUDGET;
    if (cfg->n_steps < 1 || cfg->switch_step < 0 || cfg->switch_step > cfg->n_steps) return BSATTN_ERR_BUDGET;
    if (!budget_valid(cfg->budget_first) || !budget_valid(cfg->budget_later)) return BSATTN_ERR_BUDGET;
    bsattn_stage* st = new (std::nothrow) bsattn_stage();
    if (st == nullptr) return BSATTN_ERR_UNSUPPORTED;
    st->cfg = *cfg;
    st->cfg.exclude = nullptr;                 // the list is copied, the pointer is not kept
    st->exclude = split_list(cfg->exclude);
    *out = st;
    return BSATTN_OK;
}

void bsattn_stage_destroy(bsattn_stage* stage) { delete stage; }

bsattn_status bsattn_stage_decide(bsattn_stage* stage, const bsattn_stage_call* call,
                                  bsattn_stage_decision* out) {
    if (stage == nullptr || call == nullptr || out == nullptr) return BSATTN_ERR_NULL;
    if (call->q_len < 0 || call->kv_len < 0 || call->step < 0) return BSATTN_ERR_SHAPE;
    const bsattn_stage_config& c = stage->cfg;
    std::lock_guard<std::mutex> guard(stage->lock);

    int32_t outcome = BSATTN_STAGE_SPARSE;
    if (!c.enabled) {
        outcome = BSATTN_DECLINE_DISABLED;
    } else if (!c.backend_block_mask) {
        outcome = BSATTN_DECLINE_NO_BACKEND;
    } else {
        const auto key = std::make_tuple(lower_trim(call->architecture ? call->architecture : ""),
                                         lower_trim(call->pipeline ? call->pipeline : ""),
                                         lower_trim(call->denoiser ? call->denoiser : ""));
        auto it = stage->excluded.find(key);
        if (it == stage->excluded.end()) {
            bool hit = false;
            for (const std::string& e : stage->exclude)
                hit = hit || e == std::get<0>(key) || e == std::get<1>(key) || e == std::get<2>(key);
            it = stage->excluded.emplace(key, hit).first;
        }
        if (it->second) outcome = BSATTN_DECLINE_EXCLUDED;
        else if (!call->self_attention || call->q_len != call->kv_len) outcome = BSATTN_DECLINE_NOT_SELF;
        else if (c.min_length > 0 && call->q_len < c.min_length) outcome = BSATTN_DECLINE_SHORT;
        else if (call->causal) outcome = BSATTN_DECLINE_CAUSAL;
        else if (call->has_token_mask && !c.backend_masked_block) outcome = BSATTN_DECLINE_TOKEN_MASK;
    }

    out->outcome = outcome;
    out->note = (outcome == BSATTN_STAGE_SPARSE && !call->has_layout) ? BSATTN_NOTE_NO_LAYOUT : BSATTN_NOTE_NONE;
    out->budget = 0.0;
    out->use_key_mask = 0;
    if (outcome == BSATTN_STAGE_SPARSE) {
        const int32_t step = call->step < c.n_steps ? call->step : c.n_steps - 1;
        out->budget = step < c.switch_step ? c.budget_first : c.budget_later;
        out->use_key_mask = call->has_token_mask ? 1 : 0;
    }
    // report once per (outcome, note, length); a served call with a layout is
    // the quiet normal case and is never reported
    out->first_report = 0;
    if (outcome != BSATTN_STAGE_SPARSE || out->note != BSATTN_NOTE_NONE) {
        const auto rk = std::make_tuple(outcome, out->note, call->q_len);
        out->first_report = stage->reported.insert(rk).second ? 1 : 0;
    }
    return BSATTN_OK;
}

}  // extern "C"
